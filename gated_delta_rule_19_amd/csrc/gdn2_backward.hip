// Backward pass of the chunked GDN-2 forward on gfx950.
//
// The gradient of the per-token recurrence of the burn-gdn2 0.1.9 README
// ("Architecture") is fixed by the forward; the README calls the chunked WY
// mode the training mode.  The backward follows the chunk structure of the
// forward (notation of the chunk kernels: per chunk of 64 tokens entering
// with state S0, Gamma = cumulative key-axis decay, Qh = Gamma q,
// Eh = Gamma (b k), Ktil_s = k_s Gamma_L / Gamma_s, A and P the decayed
// key-key and query-key products, T = (I + A)^{-1}, W = T Eh, U = T (w v),
// Delta = U - W S0, O = Qh S0 + P Delta, S_L = Gamma_L S0 + Ktil^T Delta):
//
//   launch 1-2  the forward prep and state pass, the state pass writing the
//               state entering every chunk (fp32 checkpoints);
//   launch 3    k_chunk_state_bwd: chunks in reverse, per (batch, head, value
//               slice), carrying the gradient dS of the chunk's exit state:
//                 dDelta = P^T dO + Ktil dS
//                 dS     = Qh^T dO + Gamma_L dS - W^T dDelta
//               writing the dS each chunk receives; what is left is dS0;
//   launch 4    k_chunk_grad: every chunk in parallel, from its entry state
//               S0, its exit gradient dSL and dO, recomputes the chunk's
//               factors in fp32 from the inputs and forms
//                 Delta, dDelta, dQh = dO S0^T, dP = mask(dO Delta^T),
//                 dKtil = Delta dSL^T, dGamma_L = rowsum(dSL * S0),
//                 dW = -dDelta S0^T, du = T^T dDelta, dT = dDelta u^T + dW Eh^T,
//                 dEh = T^T dW, dA = mask(-T^T dT T^T),
//               then the gradients of q, k, b and of the cumulative log decay
//               through the definitions of Qh, Eh, Ktil, A and P, and
//               dalpha from the reverse cumulative sum of the latter.
//
// Decay ratios Gamma_r / Gamma_s (s <= r) inside A, P and their gradients
// are split at the first token j0 of s's 16-token block:
// exp(G_r - G_s) = exp(G_r - G_j0) * exp(G_j0 - G_s), the first factor <= 1
// on the row side, the second >= 1 but bounded by the decay domain of the
// chunked mode (products of alpha over 16 tokens above ~1e-30) on the
// column side, so every one of them is a plain product per column block.
//
// This first version computes with fp32 vector FMAs: a generic product on
// 256 threads stages K-slices of both operands in LDS and keeps 4x4 output
// tiles in registers, and the per-chunk intermediates live in a global
// scratch area per workgroup (cache resident).
#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"
#include "gdn2_layout.hpp"

namespace gdn2 {

// ---------------------------------------------------------------------------
// C[M][N] = sum_k A(m, k) B(k, n) on the 256 threads of a workgroup.
// M, N multiples of 4 with M <= 128, N <= 256, M * N <= 16384; any K.
// fa(m, k) and fb(k, n) return operand elements (fp32); fe(m, n, v) consumes
// each result.  Ends with a barrier, so the next product may read what fe
// wrote.
// ---------------------------------------------------------------------------
constexpr int kGK = 16;
struct __attribute__((aligned(16))) GemmLds {
    float a[kGK][128];
    float b[kGK][256];
};

template <typename FA, typename FB, typename FE>
__device__ void gemm(GemmLds& sm, int M, int N, int K, FA fa, FB fb, FE fe)
{
    const int tid = threadIdx.x;
    const int tnc = N / 4, nsl = (M / 4) * tnc;
    // passes of up to 512 4x4 tiles (two per thread); larger products
    // stage their operands once per pass
    for (int p0 = 0; p0 < nsl; p0 += 2 * kThreads) {
        float acc[2][4][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[t][i][j] = 0.f;
        for (int k0 = 0; k0 < K; k0 += kGK) {
            for (int i = tid; i < M * kGK; i += kThreads) {
                const int m = i / kGK, kk = i - m * kGK;
                sm.a[kk][m] = k0 + kk < K ? fa(m, k0 + kk) : 0.f;
            }
            for (int i = tid; i < kGK * N; i += kThreads) {
                const int kk = i / N, n = i - kk * N;
                sm.b[kk][n] = k0 + kk < K ? fb(k0 + kk, n) : 0.f;
            }
            __syncthreads();
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int slot = p0 + tid + t * kThreads;
                if (slot < nsl) {
                    const int m0 = 4 * (slot / tnc), n0 = 4 * (slot - (slot / tnc) * tnc);
#pragma unroll 4
                    for (int kk = 0; kk < kGK; ++kk) {
                        const f32x4 av = *reinterpret_cast<const f32x4*>(&sm.a[kk][m0]);
                        const f32x4 bv = *reinterpret_cast<const f32x4*>(&sm.b[kk][n0]);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < 4; ++j) acc[t][i][j] += av[i] * bv[j];
                    }
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int slot = p0 + tid + t * kThreads;
            if (slot < nsl) {
                const int m0 = 4 * (slot / tnc), n0 = 4 * (slot - (slot / tnc) * tnc);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) fe(m0 + i, n0 + j, acc[t][i][j]);
            }
        }
    }
    __syncthreads();
}

template <typename T> __device__ inline float ldf(const T* p, int64_t i) { return Io<T>::to_f(p[i]); }
template <typename T> __device__ inline void stf(T* p, int64_t i, float x) { p[i] = Io<T>::from_f(x); }

// ---------------------------------------------------------------------------
// launch 3: reverse pass over chunks
// ---------------------------------------------------------------------------
template <typename Tio>
__global__ __launch_bounds__(kThreads) void k_chunk_state_bwd(BwdStateArgs a)
{
    __shared__ GemmLds gl;
    __shared__ float dS[128 * 64];     // [dk][vs]
    __shared__ float dD[64 * 64];      // [64][vs]
    const int tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv, vs = a.vs, nt = a.nt;
    const int64_t chain = blockIdx.x / a.nslices;
    const int j0 = (int)(blockIdx.x - chain * a.nslices) * vs;
    const int64_t bb = chain / a.H, hh = chain - bb * a.H;
    const int kb = sizeof(Tio) == 2 ? 32 : 16;
    const WsLayout LY = ws_layout(dk, dv, sizeof(Tio), kb);
    const int kpad = (dk + kb - 1) / kb * kb;
    const Tio* dO = static_cast<const Tio*>(a.dO);

    for (int i = tid; i < dk * vs; i += kThreads) {
        const int c = i / vs, j = i - c * vs;
        dS[i] = a.dS_T ? a.dS_T[(chain * dk + c) * dv + j0 + j] : 0.f;
    }
    __syncthreads();
    for (int n = nt - 1; n >= 0; --n) {
        const char* blk = static_cast<const char*>(a.ws) + (chain * nt + n) * a.ws_block;
        const Tio* Qh = reinterpret_cast<const Tio*>(blk + LY.qh);
        const Tio* Wf = reinterpret_cast<const Tio*>(blk + LY.wwy);
        const Tio* Ktt = reinterpret_cast<const Tio*>(blk + LY.ktt);
        const Tio* Pf = reinterpret_cast<const Tio*>(blk + LY.p);
        const float* gam = reinterpret_cast<const float*>(blk + LY.gaml);
        const int64_t t0 = (int64_t)n * kChunk;
        const int L = (int)(a.T - t0 < kChunk ? a.T - t0 : kChunk);
        auto dOf = [&](int r, int j) -> float {
            return r < L ? ldf(dO, ((bb * a.T + t0 + r) * a.H + hh) * dv + j0 + j) : 0.f;
        };
        // the gradient this chunk's exit state receives
        float* dsl = a.dSL + (chain * nt + n) * (int64_t)dk * dv + j0;
        for (int i = tid; i < dk * vs; i += kThreads) {
            const int c = i / vs, j = i - c * vs;
            dsl[(int64_t)c * dv + j] = dS[i];
        }
        // dDelta = P^T dO + Ktil dS
        gemm(gl, 64, vs, 64 + dk,
             [&](int m, int k) { return k < 64 ? ldf(Pf, k * 64 + m) : ldf(Ktt, (k - 64) * 64 + m); },
             [&](int k, int j) { return k < 64 ? dOf(k, j) : dS[(k - 64) * vs + j]; },
             [&](int m, int j, float v) { dD[m * vs + j] = v; });
        // dS = Qh^T dO - W^T dDelta + Gamma_L dS
        gemm(gl, dk, vs, 128,
             [&](int m, int k) { return k < 64 ? ldf(Qh, k * kpad + m) : -ldf(Wf, (k - 64) * kpad + m); },
             [&](int k, int j) { return k < 64 ? dOf(k, j) : dD[(k - 64) * vs + j]; },
             [&](int m, int j, float v) { dS[m * vs + j] = v + gam[m] * dS[m * vs + j]; });
    }
    if (a.dS0 != nullptr) {
        for (int i = tid; i < dk * vs; i += kThreads) {
            const int c = i / vs, j = i - c * vs;
            a.dS0[(chain * dk + c) * dv + j0 + j] = dS[i];
        }
    }
}

// ---------------------------------------------------------------------------
// launch 4: per-chunk gradients
// ---------------------------------------------------------------------------
// fp32 scratch of one workgroup, in floats
__host__ __device__ inline int64_t grad_scratch_floats(int dk, int dv)
{
    return 17 * 64 * (int64_t)dk + 5 * 64 * (int64_t)dv + 7 * 64 * 64 + dk;
}

template <typename Tio, typename Tg>
__global__ __launch_bounds__(kThreads) void k_chunk_grad(GradArgs a)
{
    __shared__ GemmLds gl;
    const int tid = threadIdx.x;
    const int dk = a.dk, dv = a.dv, nt = a.nt;
    const int KA = 64 * dk, VA = 64 * dv, QA = 64 * 64;
    float* sc = a.scratch + blockIdx.x * grad_scratch_floats(dk, dv);
    // 64 x dk arrays
    float *G = sc, *Qh = G + KA, *Eh = Qh + KA, *Kt = Eh + KA, *KY = Kt + KA, *qf = KY + KA, *kf = qf + KA;
    float *ef = kf + KA, *W = ef + KA, *dQh = W + KA, *dKt = dQh + KA, *dW = dKt + KA, *dEh = dW + KA;
    float *deA = dEh + KA, *dqP = deA + KA, *dkA = dqP + KA, *dkP = dkA + KA;
    // 64 x dv arrays
    float *u = dkP + KA, *dOf = u + VA, *U = dOf + VA, *Dl = U + VA, *dDl = Dl + VA;
    // 64 x 64 arrays
    float *A = dDl + VA, *P = A + QA, *Tm = P + QA, *dP = Tm + QA, *dT = dP + QA, *tmp = dT + QA, *dA = tmp + QA;
    float* dGamL = dA + QA;

    const Tio* q = static_cast<const Tio*>(a.q);
    const Tio* k = static_cast<const Tio*>(a.k);
    const Tio* v = static_cast<const Tio*>(a.v);
    const Tio* dO = static_cast<const Tio*>(a.dO);
    const Tg* alpha = static_cast<const Tg*>(a.alpha);
    const Tg* bg = static_cast<const Tg*>(a.b);
    const Tg* wg = static_cast<const Tg*>(a.w);
    Tio* dq = static_cast<Tio*>(a.dq);
    Tio* dk_out = static_cast<Tio*>(a.dk_out);
    Tio* dv_out = static_cast<Tio*>(a.dv_out);
    Tg* dalpha = static_cast<Tg*>(a.dalpha);
    Tg* db = static_cast<Tg*>(a.db);
    Tg* dw = static_cast<Tg*>(a.dw);

    for (int64_t ci = blockIdx.x; ci < a.total; ci += gridDim.x) {
        const int64_t chain = ci / nt;
        const int n = (int)(ci - chain * nt);
        const int64_t bb = chain / a.H, hh = chain - bb * a.H;
        const int64_t t0 = (int64_t)n * kChunk;
        const int L = (int)(a.T - t0 < kChunk ? a.T - t0 : kChunk);
        const int64_t row0 = (bb * a.T + t0) * a.H + hh;        // row of token t0
        const int64_t H = a.H;
        const float* S0 = a.S_chk + ci * (int64_t)dk * dv;      // [dk][dv]
        const float* dSL = a.dSL + ci * (int64_t)dk * dv;

        // ---- G: cumulative log decay (padding tokens have alpha = 1)
        for (int c = tid; c < dk; c += kThreads) {
            float g = 0.f;
            for (int r = 0; r < 64; ++r) {
                if (r < L) g += __logf(ldf(alpha, (row0 + r * H) * dk + c));
                G[r * dk + c] = g;
            }
        }
        __syncthreads();
        // ---- decay-scaled operands; zero the accumulated arrays
        for (int i = tid; i < KA; i += kThreads) {
            const int r = i / dk, c = i - r * dk;
            const bool ok = r < L;
            const int64_t src = (row0 + r * H) * dk + c;
            const float qv = ok ? ldf(q, src) : 0.f, kv = ok ? ldf(k, src) : 0.f, bv = ok ? ldf(bg, src) : 0.f;
            const float g = G[i], gam = __expf(g);
            qf[i] = qv;
            kf[i] = kv;
            ef[i] = bv * kv;
            Qh[i] = gam * qv;
            Eh[i] = gam * bv * kv;
            Kt[i] = kv * __expf(G[63 * dk + c] - g);
            KY[i] = kv * __expf(G[(r & ~15) * dk + c] - g);
            deA[i] = dqP[i] = dkA[i] = dkP[i] = 0.f;
        }
        for (int i = tid; i < VA; i += kThreads) {
            const int r = i / dv, j = i - r * dv;
            const bool ok = r < L;
            const int64_t src = (row0 + r * H) * dv + j;
            u[i] = ok ? ldf(wg, src) * ldf(v, src) : 0.f;
            dOf[i] = ok ? ldf(dO, src) : 0.f;
        }
        for (int i = tid; i < QA; i += kThreads) A[i] = P[i] = Tm[i] = 0.f;
        __syncthreads();

        // ---- A (s < r) and P (s <= r), one 16-column block at a time
        for (int J = 0; J < 4; ++J) {
            const int j0 = 16 * J;
            gemm(gl, 64 - j0, 16, dk,
                 [&](int m, int c) { return ef[(j0 + m) * dk + c] * __expf(G[(j0 + m) * dk + c] - G[j0 * dk + c]); },
                 [&](int c, int s) { return KY[(j0 + s) * dk + c]; },
                 [&](int m, int s, float x) { if (s < m) A[(j0 + m) * 64 + j0 + s] = x; });
            gemm(gl, 64 - j0, 16, dk,
                 [&](int m, int c) { return qf[(j0 + m) * dk + c] * __expf(G[(j0 + m) * dk + c] - G[j0 * dk + c]); },
                 [&](int c, int s) { return KY[(j0 + s) * dk + c]; },
                 [&](int m, int s, float x) { if (s <= m) P[(j0 + m) * 64 + j0 + s] = x; });
        }

        // ---- T = (I + A)^{-1}: diagonal 16x16 blocks by substitution (one wave
        // each, lane = column), then the block rows below
        {
            const int wv = tid >> 6, c = tid & 63;
            if (c < 16) {
                const int o = 16 * wv;
                float col[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float x = (i == c) ? 1.f : 0.f;
#pragma unroll
                    for (int s = 0; s < 16; ++s)
                        if (s < i) x -= A[(o + i) * 64 + o + s] * col[s];
                    col[i] = (i < c) ? 0.f : x;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) Tm[(o + i) * 64 + o + c] = col[i];
            }
        }
        __syncthreads();
        for (int I = 1; I < 4; ++I) {
            // tmp[J] = sum_{K=J}^{I-1} A_IK T_KJ  for J < I
            for (int e = tid; e < I * 256; e += kThreads) {
                const int J = e >> 8, i = (e >> 4) & 15, c = e & 15;
                float x = 0.f;
                for (int s = 16 * J; s < 16 * I; ++s) x += A[(16 * I + i) * 64 + s] * Tm[s * 64 + 16 * J + c];
                tmp[J * 256 + i * 16 + c] = x;
            }
            __syncthreads();
            for (int e = tid; e < I * 256; e += kThreads) {
                const int J = e >> 8, i = (e >> 4) & 15, c = e & 15;
                float x = 0.f;
                for (int s = 0; s <= i; ++s) x += Tm[(16 * I + i) * 64 + 16 * I + s] * tmp[J * 256 + s * 16 + c];
                Tm[(16 * I + i) * 64 + 16 * J + c] = -x;
            }
            __syncthreads();
        }

        // ---- U = T u, W = T Eh
        gemm(gl, 64, dv, 64, [&](int m, int s) { return Tm[m * 64 + s]; }, [&](int s, int j) { return u[s * dv + j]; },
             [&](int m, int j, float x) { U[m * dv + j] = x; });
        gemm(gl, 64, dk, 64, [&](int m, int s) { return Tm[m * 64 + s]; }, [&](int s, int c) { return Eh[s * dk + c]; },
             [&](int m, int c, float x) { W[m * dk + c] = x; });
        // ---- Delta = U - W S0;  dDelta = P^T dO + Ktil dSL
        gemm(gl, 64, dv, dk, [&](int m, int c) { return W[m * dk + c]; },
             [&](int c, int j) { return S0[(int64_t)c * dv + j]; },
             [&](int m, int j, float x) { Dl[m * dv + j] = U[m * dv + j] - x; });
        gemm(gl, 64, dv, 64 + dk,
             [&](int m, int kk) { return kk < 64 ? P[kk * 64 + m] : Kt[m * dk + kk - 64]; },
             [&](int kk, int j) { return kk < 64 ? dOf[kk * dv + j] : dSL[(int64_t)(kk - 64) * dv + j]; },
             [&](int m, int j, float x) { dDl[m * dv + j] = x; });
        // ---- dQh, dP, dKtil, dW, du (-> dw, dv), dGamma_L
        gemm(gl, 64, dk, dv, [&](int m, int j) { return dOf[m * dv + j]; },
             [&](int j, int c) { return S0[(int64_t)c * dv + j]; }, [&](int m, int c, float x) { dQh[m * dk + c] = x; });
        gemm(gl, 64, 64, dv, [&](int m, int j) { return dOf[m * dv + j]; }, [&](int j, int s) { return Dl[s * dv + j]; },
             [&](int m, int s, float x) { dP[m * 64 + s] = s <= m ? x : 0.f; });
        gemm(gl, 64, dk, dv, [&](int m, int j) { return Dl[m * dv + j]; },
             [&](int j, int c) { return dSL[(int64_t)c * dv + j]; }, [&](int m, int c, float x) { dKt[m * dk + c] = x; });
        gemm(gl, 64, dk, dv, [&](int m, int j) { return dDl[m * dv + j]; },
             [&](int j, int c) { return S0[(int64_t)c * dv + j]; }, [&](int m, int c, float x) { dW[m * dk + c] = -x; });
        gemm(gl, 64, dv, 64, [&](int m, int s) { return Tm[s * 64 + m]; }, [&](int s, int j) { return dDl[s * dv + j]; },
             [&](int r, int j, float x) {
                 if (r < L) {
                     const int64_t o = (row0 + r * H) * dv + j;
                     stf(dw, o, x * ldf(v, o));
                     stf(dv_out, o, x * ldf(wg, o));
                 }
             });
        for (int c = tid; c < dk; c += kThreads) {
            float x = 0.f;
            for (int j = 0; j < dv; ++j) x += dSL[(int64_t)c * dv + j] * S0[(int64_t)c * dv + j];
            dGamL[c] = x;
        }
        // ---- dT = dDelta u^T + dW Eh^T, dEh = T^T dW, dA = mask(-T^T dT T^T)
        gemm(gl, 64, 64, dv + dk,
             [&](int m, int kk) { return kk < dv ? dDl[m * dv + kk] : dW[m * dk + kk - dv]; },
             [&](int kk, int s) { return kk < dv ? u[s * dv + kk] : Eh[s * dk + kk - dv]; },
             [&](int m, int s, float x) { dT[m * 64 + s] = x; });
        gemm(gl, 64, dk, 64, [&](int m, int s) { return Tm[s * 64 + m]; }, [&](int s, int c) { return dW[s * dk + c]; },
             [&](int m, int c, float x) { dEh[m * dk + c] = x; });
        gemm(gl, 64, 64, 64, [&](int m, int s) { return Tm[s * 64 + m]; }, [&](int s, int j) { return dT[s * 64 + j]; },
             [&](int m, int j, float x) { tmp[m * 64 + j] = x; });
        gemm(gl, 64, 64, 64, [&](int m, int j) { return tmp[m * 64 + j]; }, [&](int j, int s) { return Tm[s * 64 + j]; },
             [&](int m, int s, float x) { dA[m * 64 + s] = s < m ? -x : 0.f; });

        // ---- through A and P: row side (rows r >= j0 of column block J) and
        // column side (columns s of block J)
        for (int J = 0; J < 4; ++J) {
            const int j0 = 16 * J;
            gemm(gl, 64 - j0, dk, 16, [&](int m, int s) { return dA[(j0 + m) * 64 + j0 + s]; },
                 [&](int s, int c) { return KY[(j0 + s) * dk + c]; },
                 [&](int m, int c, float x) {
                     const int r = j0 + m;
                     deA[r * dk + c] += x * __expf(G[r * dk + c] - G[j0 * dk + c]);
                 });
            gemm(gl, 64 - j0, dk, 16, [&](int m, int s) { return dP[(j0 + m) * 64 + j0 + s]; },
                 [&](int s, int c) { return KY[(j0 + s) * dk + c]; },
                 [&](int m, int c, float x) {
                     const int r = j0 + m;
                     dqP[r * dk + c] += x * __expf(G[r * dk + c] - G[j0 * dk + c]);
                 });
            gemm(gl, 16, dk, 64 - j0, [&](int m, int rr) { return dA[(j0 + rr) * 64 + j0 + m]; },
                 [&](int rr, int c) {
                     const int r = j0 + rr;
                     return ef[r * dk + c] * __expf(G[r * dk + c] - G[j0 * dk + c]);
                 },
                 [&](int m, int c, float x) {
                     const int s = j0 + m;
                     dkA[s * dk + c] += x * __expf(G[j0 * dk + c] - G[s * dk + c]);
                 });
            gemm(gl, 16, dk, 64 - j0, [&](int m, int rr) { return dP[(j0 + rr) * 64 + j0 + m]; },
                 [&](int rr, int c) {
                     const int r = j0 + rr;
                     return qf[r * dk + c] * __expf(G[r * dk + c] - G[j0 * dk + c]);
                 },
                 [&](int m, int c, float x) {
                     const int s = j0 + m;
                     dkP[s * dk + c] += x * __expf(G[j0 * dk + c] - G[s * dk + c]);
                 });
        }

        // ---- gradients of q, k, b and of G (dG kept in deA's place)
        for (int i = tid; i < KA; i += kThreads) {
            const int r = i / dk, c = i - r * dk;
            const float g = G[i], gam = __expf(g);
            const float de = gam * dEh[i] + deA[i];
            const float kv = kf[i];
            const bool ok = r < L;
            const int64_t o = (row0 + r * H) * dk + c;
            const float bv = ok ? ldf(bg, o) : 0.f;
            const float dG = dQh[i] * Qh[i] + dEh[i] * Eh[i] - dKt[i] * Kt[i] + ef[i] * deA[i] + qf[i] * dqP[i] -
                             kv * (dkA[i] + dkP[i]);
            if (ok) {
                stf(dq, o, gam * dQh[i] + dqP[i]);
                stf(dk_out, o, __expf(G[63 * dk + c] - g) * dKt[i] + dkA[i] + dkP[i] + de * bv);
                stf(db, o, de * kv);
            }
            deA[i] = dG;
        }
        __syncthreads();
        // dG at the last token also carries Gamma_L's uses; dlog(alpha) is the
        // reverse cumulative sum of dG
        for (int c = tid; c < dk; c += kThreads) {
            float extra = dGamL[c] * __expf(G[63 * dk + c]);
            for (int r = 0; r < 64; ++r) extra += dKt[r * dk + c] * Kt[r * dk + c];
            float acc = extra;
            for (int r = 63; r >= 0; --r) {
                acc += deA[r * dk + c];
                if (r < L) {
                    const int64_t o = (row0 + r * H) * dk + c;
                    stf(dalpha, o, acc / ldf(alpha, o));
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int64_t grad_blocks(int64_t total) { return total < 1024 ? total : 1024; }

int64_t chunk_grad_scratch_bytes(int dk, int dv, int64_t total)
{
    return grad_blocks(total) * grad_scratch_floats(dk, dv) * 4;
}

hipError_t launch_chunk_state_bwd(const BwdStateArgs& a, bool bf16, hipStream_t s)
{
    const int64_t nblk = a.B * a.H * (int64_t)a.nslices;
    if (bf16)
        hipLaunchKernelGGL(k_chunk_state_bwd<__bf16>, dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(k_chunk_state_bwd<float>, dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_chunk_grad(const GradArgs& a, bool bf16, bool gbf16, hipStream_t s)
{
    const dim3 grid((unsigned)grad_blocks(a.total));
    if (!bf16) {
        if (gbf16) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_chunk_grad<float, float>), grid, dim3(kThreads), 0, s, a);
    } else if (gbf16) {
        hipLaunchKernelGGL((k_chunk_grad<__bf16, __bf16>), grid, dim3(kThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL((k_chunk_grad<__bf16, float>), grid, dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace gdn2
