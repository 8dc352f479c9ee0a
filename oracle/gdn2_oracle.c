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

/*
 * Gradient of the same recurrence (fp64, TEST INFRASTRUCTURE): for output
 * gradients dO [B,T,H,dv] and dS_T [B,H,dk,dv] (nullable = 0) it returns the
 * derivative of  sum(dO * o) + sum(dS_T * S_T)  with respect to q, k, v,
 * alpha, b, w (same layouts as the inputs) and S0 (dS0 [B,H,dk,dv]).  The
 * README prints no gradient; the gradient of a function is unique, so this is
 * the reverse of the five steps above, token by token.  With z = alpha*b*k,
 * u = w*v one step is S_t = diag(alpha) S_{t-1} + k delta^T with
 * delta = u - S_{t-1}^T z, and with G the gradient of S_t:
 *     G      += q dO_t^T              dq    = S_t dO_t
 *     ddelta  = G^T k                 dk    = G delta + dz * alpha * b
 *     dz      = -S_{t-1} ddelta       dw    = ddelta * v,  dv = ddelta * w
 *     db      = dz * alpha * k        dalpha = rowsum(G * S_{t-1}) + dz * b * k
 *     G      <- diag(alpha) G - z ddelta^T      (dS0 = G after token 0)
 * then through the prologue flags: a logit gate g = s * sigmoid(x) gives
 * dx = dg * s * sigmoid(x) (1 - sigmoid(x)); the norm x_hat = x r,
 * r = (|x|^2 + 1e-6)^(-1/2), gives dx = r (dx_hat - x_hat (x_hat . dx_hat)).
 * Each (batch, head) chain runs on one thread: a forward pass keeps the state
 * at every 64th token, then each 64-token span is replayed from its
 * checkpoint before it is reversed.  Returns 0, or -1 on bad sizes or when
 * memory runs out.
 */
int gdn2_oracle_bwd_f64(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                        const float* q, const float* k, const float* v,
                        const float* alpha, const float* b, const float* w,
                        const float* S0, const float* dO, const float* dS_T,
                        double* dq, double* dk_out, double* dv_out,
                        double* dalpha, double* db, double* dw, double* dS0,
                        int nthreads, int flags)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    const int64_t span = 64;
    const int64_t nspan = (T + span - 1) / span;
    const int64_t units = B * H;
    const int64_t SZ = dk * dv;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        double* ck = (double*)malloc(sizeof(double) * (size_t)((nspan + 1) * SZ));   /* state entering each span */
        double* Sb = (double*)malloc(sizeof(double) * (size_t)((span + 1) * SZ));    /* states inside one span */
        double* G = (double*)malloc(sizeof(double) * (size_t)SZ);
        double* vec = (double*)malloc(sizeof(double) * (size_t)(12 * dk + 8 * dv));
        if (!ck || !Sb || !G || !vec) {
#pragma omp atomic write
            failed = 1;
        }
        /* one token's prologue-mapped inputs and work vectors */
        double *qa = vec, *ka = vec + dk, *aa = vec + 2 * dk, *ba = vec + 3 * dk, *za = vec + 4 * dk;
        double *gq = vec + 5 * dk, *gk = vec + 6 * dk, *ga = vec + 7 * dk, *gb = vec + 8 * dk, *dz = vec + 9 * dk;
        double *sq_raw = vec + 10 * dk, *sk_raw = vec + 11 * dk;
        double *ua = vec + 12 * dk, *wa = ua + dv, *del = wa + dv, *dd = del + dv, *gw = dd + dv, *gv = gw + dv;
        double *r = gv + dv, *dOa = r + dv;
        double nrm[2];

        /* token t of chain (bi, hi): inputs after the prologue into qa, ka, aa, ba, wa, ua, za;
           nrm = the q and k scales r (1 without the norm) */
#define LOAD_TOKEN(t)                                                                         \
    do {                                                                                      \
        const int64_t kb_ = ((bi * T + (t)) * H + hi) * dk, vb_ = ((bi * T + (t)) * H + hi) * dv; \
        double nq_ = 0.0, nk_ = 0.0;                                                          \
        for (int64_t c = 0; c < dk; ++c) {                                                    \
            qa[c] = (double)q[kb_ + c];                                                       \
            ka[c] = (double)k[kb_ + c];                                                       \
            sq_raw[c] = qa[c];                                                                \
            sk_raw[c] = ka[c];                                                                \
            nq_ += qa[c] * qa[c];                                                             \
            nk_ += ka[c] * ka[c];                                                             \
            aa[c] = (double)alpha[kb_ + c];                                                   \
            ba[c] = (double)b[kb_ + c];                                                       \
            if (flags & 1) {                                                                  \
                aa[c] = logistic(aa[c]);                                                      \
                ba[c] = logistic(ba[c]) * ((flags & 2) ? 2.0 : 1.0);                          \
            }                                                                                 \
        }                                                                                     \
        nrm[0] = nrm[1] = 1.0;                                                                \
        if (flags & 4) {                                                                      \
            nrm[0] = 1.0 / sqrt(nq_ + 1e-6);                                                  \
            nrm[1] = 1.0 / sqrt(nk_ + 1e-6);                                                  \
            for (int64_t c = 0; c < dk; ++c) {                                                \
                qa[c] *= nrm[0];                                                              \
                ka[c] *= nrm[1];                                                              \
            }                                                                                 \
        }                                                                                     \
        for (int64_t c = 0; c < dk; ++c) za[c] = aa[c] * ba[c] * ka[c];                       \
        for (int64_t j = 0; j < dv; ++j) {                                                    \
            wa[j] = (double)w[vb_ + j];                                                       \
            if (flags & 1) wa[j] = logistic(wa[j]);                                           \
            ua[j] = wa[j] * (double)v[vb_ + j];                                               \
        }                                                                                     \
    } while (0)

        /* S_next = diag(alpha) S + k (u - S^T z)^T  (the same step as the forward above) */
#define STEP(Sin, Sout)                                                                       \
    do {                                                                                      \
        for (int64_t j = 0; j < dv; ++j) r[j] = 0.0;                                          \
        for (int64_t c = 0; c < dk; ++c)                                                      \
            for (int64_t j = 0; j < dv; ++j) r[j] += za[c] * (Sin)[c * dv + j];               \
        for (int64_t c = 0; c < dk; ++c)                                                      \
            for (int64_t j = 0; j < dv; ++j)                                                  \
                (Sout)[c * dv + j] = aa[c] * (Sin)[c * dv + j] + ka[c] * (ua[j] - r[j]);      \
    } while (0)

#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (failed) continue;
            const int64_t bi = u / H, hi = u % H;
            const int64_t sb = (bi * H + hi) * SZ;
            /* forward: checkpoints */
            for (int64_t e = 0; e < SZ; ++e) ck[e] = S0 ? (double)S0[sb + e] : 0.0;
            for (int64_t n = 0; n < nspan; ++n) {
                double* cur = Sb;
                memcpy(cur, ck + n * SZ, sizeof(double) * (size_t)SZ);
                const int64_t t1 = (n + 1) * span < T ? (n + 1) * span : T;
                for (int64_t t = n * span; t < t1; ++t) {
                    LOAD_TOKEN(t);
                    double* nxt = (cur == Sb) ? Sb + SZ : Sb;
                    STEP(cur, nxt);
                    cur = nxt;
                }
                memcpy(ck + (n + 1) * SZ, cur, sizeof(double) * (size_t)SZ);
            }
            /* reverse */
            for (int64_t e = 0; e < SZ; ++e) G[e] = dS_T ? (double)dS_T[sb + e] : 0.0;
            for (int64_t n = nspan - 1; n >= 0; --n) {
                const int64_t t0 = n * span, t1 = (n + 1) * span < T ? (n + 1) * span : T;
                memcpy(Sb, ck + n * SZ, sizeof(double) * (size_t)SZ);
                for (int64_t t = t0; t < t1; ++t) {
                    LOAD_TOKEN(t);
                    STEP(Sb + (t - t0) * SZ, Sb + (t - t0 + 1) * SZ);
                }
                for (int64_t t = t1 - 1; t >= t0; --t) {
                    LOAD_TOKEN(t);
                    const double* Sp = Sb + (t - t0) * SZ;
                    const double* St = Sb + (t - t0 + 1) * SZ;
                    const int64_t kb = ((bi * T + t) * H + hi) * dk, vb = ((bi * T + t) * H + hi) * dv;
                    for (int64_t j = 0; j < dv; ++j) dOa[j] = (double)dO[vb + j];
                    /* G += q dO^T;  dq = S_t dO */
                    for (int64_t c = 0; c < dk; ++c) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < dv; ++j) {
                            G[c * dv + j] += qa[c] * dOa[j];
                            acc += St[c * dv + j] * dOa[j];
                        }
                        gq[c] = acc;
                    }
                    /* delta = u - S_{t-1}^T z;  ddelta = G^T k */
                    for (int64_t j = 0; j < dv; ++j) {
                        del[j] = ua[j];
                        dd[j] = 0.0;
                    }
                    for (int64_t c = 0; c < dk; ++c)
                        for (int64_t j = 0; j < dv; ++j) {
                            del[j] -= Sp[c * dv + j] * za[c];
                            dd[j] += G[c * dv + j] * ka[c];
                        }
                    /* dz = -S_{t-1} ddelta; dk, db, dalpha */
                    for (int64_t c = 0; c < dk; ++c) {
                        double s1 = 0.0, s2 = 0.0, s3 = 0.0;
                        for (int64_t j = 0; j < dv; ++j) {
                            s1 += Sp[c * dv + j] * dd[j];
                            s2 += G[c * dv + j] * del[j];
                            s3 += G[c * dv + j] * Sp[c * dv + j];
                        }
                        dz[c] = -s1;
                        gk[c] = s2 + dz[c] * aa[c] * ba[c];
                        gb[c] = dz[c] * aa[c] * ka[c];
                        ga[c] = s3 + dz[c] * ba[c] * ka[c];
                    }
                    for (int64_t j = 0; j < dv; ++j) {
                        gw[j] = dd[j] * (double)v[vb + j];
                        gv[j] = dd[j] * wa[j];
                    }
                    /* G <- diag(alpha) G - z ddelta^T */
                    for (int64_t c = 0; c < dk; ++c)
                        for (int64_t j = 0; j < dv; ++j) G[c * dv + j] = aa[c] * G[c * dv + j] - za[c] * dd[j];
                    /* through the prologue */
                    if (flags & 1) {
                        const double bs = (flags & 2) ? 2.0 : 1.0;
                        for (int64_t c = 0; c < dk; ++c) {
                            const double sa = aa[c], sbv = ba[c] / bs;
                            ga[c] *= sa * (1.0 - sa);
                            gb[c] *= bs * sbv * (1.0 - sbv);
                        }
                        for (int64_t j = 0; j < dv; ++j) gw[j] *= wa[j] * (1.0 - wa[j]);
                    }
                    if (flags & 4) {
                        double pq = 0.0, pk = 0.0;
                        for (int64_t c = 0; c < dk; ++c) {
                            pq += qa[c] * gq[c];
                            pk += ka[c] * gk[c];
                        }
                        for (int64_t c = 0; c < dk; ++c) {
                            gq[c] = nrm[0] * (gq[c] - qa[c] * pq);
                            gk[c] = nrm[1] * (gk[c] - ka[c] * pk);
                        }
                    }
                    for (int64_t c = 0; c < dk; ++c) {
                        dq[kb + c] = gq[c];
                        dk_out[kb + c] = gk[c];
                        dalpha[kb + c] = ga[c];
                        db[kb + c] = gb[c];
                    }
                    for (int64_t j = 0; j < dv; ++j) {
                        dw[vb + j] = gw[j];
                        dv_out[vb + j] = gv[j];
                    }
                }
            }
            for (int64_t e = 0; e < SZ; ++e) dS0[sb + e] = G[e];
        }
#undef LOAD_TOKEN
#undef STEP
        free(ck);
        free(Sb);
        free(G);
        free(vec);
    }
    return failed ? -1 : 0;
}
