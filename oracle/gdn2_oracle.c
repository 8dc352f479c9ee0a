/*
 * fp64 CPU oracle for the Gated DeltaNet-2 token mixer -- TEST INFRASTRUCTURE.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * load this library.  It shares no code with the GPU library.
 *
 * It computes the per-token recurrence of the burn-gdn2 0.1.9 README
 * (docs.rs), section "Architecture":
 *
 *     S_t = (I - k_t (b_t*k_t)^T) diag(alpha_t) S_{t-1} + k_t (w_t*v_t)^T
 *     o_t = q_t^T S_t
 *
 * in the literal order of that formula, per head and token:
 *   1. X = diag(alpha_t) S           (decay each key row c by alpha_t[c])
 *   2. r = (b_t*k_t)^T X             (the erase reads the decayed state)
 *   3. X = X - k_t r^T               ((I - k e^T) X = X - k (e^T X))
 *   4. S = X + k_t (w_t*v_t)^T       (write)
 *   5. o_t = q_t^T S                 (output reads the updated state)
 * Step 3 uses (I - k e^T) X = X - k (e^T X), which is exact in real
 * arithmetic; it avoids forming the d_k x d_k matrix.
 *
 * Value columns never mix (every gate acts on the key axis or on the written
 * row vector w*v), so the work is split over (batch, head, column block) with
 * OpenMP; the result does not depend on the split.
 *
 * Prologue flags (the library's GDN2_FLAG_* values), applied to each token's
 * inputs in double before step 1:
 *   1 gate logits: alpha = sigmoid(alpha), b = sigmoid(b), w = sigmoid(w),
 *     sigmoid(x) = 1 / (1 + exp(-x));
 *   2 with 1: b = 2 sigmoid(b) (the README's "b x 2" option);
 *   4 q and k divided by sqrt(sum over d_k of x^2 + 1e-6) per (token, head)
 *     (the README's L2-Norm before the recurrence).
 *
 * Inputs are float32 (bf16 inputs are widened exactly by the caller); all
 * arithmetic and both outputs are double.  Layouts, C-contiguous:
 *   q, k, alpha, b : [B, T, H, dk]     v, w : [B, T, H, dv]
 *   S0 (nullable = zero state), S_out : [B, H, dk, dv]     o : [B, T, H, dv]
 * Returns 0 on success, -1 on bad sizes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double logistic(double x) { return 1.0 / (1.0 + exp(-x)); }

int gdn2_oracle_f64(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                    const float* q, const float* k, const float* v,
                    const float* alpha, const float* b, const float* w,
                    const float* S0, double* o, double* S_out,
                    int nthreads, int64_t col_block, int flags)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (col_block <= 0 || col_block > dv) col_block = dv;
    const int64_t nblk = (dv + col_block - 1) / col_block;
    const int64_t units = B * H * nblk;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)(dk * col_block));
        double* r = (double*)malloc(sizeof(double) * (size_t)col_block);
        double* tk = (double*)malloc(sizeof(double) * (size_t)(4 * dk + col_block));   /* one token's inputs */
        double *qa = tk, *ka = tk + dk, *aa = tk + 2 * dk, *ba = tk + 3 * dk, *wa = tk + 4 * dk;
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            const int64_t bi = u / (H * nblk);
            const int64_t hi = (u / nblk) % H;
            const int64_t j0 = (u % nblk) * col_block;
            const int64_t nj = (j0 + col_block <= dv) ? col_block : dv - j0;

            /* state block S[:, j0:j0+nj] */
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < nj; ++j)
                    S[c * nj + j] = S0 ? (double)S0[((bi * H + hi) * dk + c) * dv + j0 + j] : 0.0;

            for (int64_t t = 0; t < T; ++t) {
                const int64_t kb = ((bi * T + t) * H + hi) * dk;   /* key-axis row */
                const int64_t vb = ((bi * T + t) * H + hi) * dv;   /* value-axis row */
                /* 0. this token's inputs, after the prologue flags */
                double nq = 0.0, nk = 0.0;
                for (int64_t c = 0; c < dk; ++c) {
                    qa[c] = (double)q[kb + c];
                    ka[c] = (double)k[kb + c];
                    aa[c] = (double)alpha[kb + c];
                    ba[c] = (double)b[kb + c];
                    nq += qa[c] * qa[c];
                    nk += ka[c] * ka[c];
                    if (flags & 1) {
                        aa[c] = logistic(aa[c]);
                        ba[c] = logistic(ba[c]) * ((flags & 2) ? 2.0 : 1.0);
                    }
                }
                if (flags & 4) {
                    const double sq = 1.0 / sqrt(nq + 1e-6), sk = 1.0 / sqrt(nk + 1e-6);
                    for (int64_t c = 0; c < dk; ++c) {
                        qa[c] *= sq;
                        ka[c] *= sk;
                    }
                }
                for (int64_t j = 0; j < nj; ++j) {
                    wa[j] = (double)w[vb + j0 + j];
                    if (flags & 1) wa[j] = logistic(wa[j]);
                }
                /* 1. decay */
                for (int64_t c = 0; c < dk; ++c) {
                    const double a = aa[c];
                    for (int64_t j = 0; j < nj; ++j) S[c * nj + j] *= a;
                }
                /* 2. r = (b*k)^T X */
                for (int64_t j = 0; j < nj; ++j) r[j] = 0.0;
                for (int64_t c = 0; c < dk; ++c) {
                    const double e = ba[c] * ka[c];
                    for (int64_t j = 0; j < nj; ++j) r[j] += e * S[c * nj + j];
                }
                /* 3. erase along k, 4. write k (w*v)^T */
                for (int64_t c = 0; c < dk; ++c) {
                    const double kc = ka[c];
                    for (int64_t j = 0; j < nj; ++j) {
                        const double uj = wa[j] * (double)v[vb + j0 + j];
                        S[c * nj + j] = (S[c * nj + j] - kc * r[j]) + kc * uj;
                    }
                }
                /* 5. o_t = q^T S_t */
                for (int64_t j = 0; j < nj; ++j) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < dk; ++c) acc += qa[c] * S[c * nj + j];
                    o[vb + j0 + j] = acc;
                }
            }
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < nj; ++j)
                    S_out[((bi * H + hi) * dk + c) * dv + j0 + j] = S[c * nj + j];
        }
        free(S);
        free(r);
        free(tk);
    }
    return 0;
}

int gdn2_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
