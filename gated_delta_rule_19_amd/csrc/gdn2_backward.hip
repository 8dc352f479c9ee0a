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
// dlog(alpha_t) gathers every term that depends on alpha_t.  Each pair (r, s)
// of A or P enters token r's row sum and token s's column sum, and the pairs
// with r, s >= t cancel in the reverse sum.  P's diagonal pairs carry no
// decay ratio and cancel inside their own token, so they are left out of
// both sums (dq and dk take them apart): every pair that is left carries a
// ratio Gamma_r / Gamma_s with s < r, of the size of what survives, and the
// fp32 sums keep their relative accuracy at fast decay.  Likewise Ktil_s
// depends on alpha_t for s < t, so its terms are summed forward from the
// chunk's first token rather than taken from a total at its last.
//
// Decay ratios Gamma_r / Gamma_s (s <= r) inside A, P and their gradients
// are split at the reference token m = 8h + 3 of s's 8-token half h, as in
// the forward: exp(G_r - G_s) = exp(G_r - G_m) * exp(G_m - G_s), each factor
// a product of decays or, within one half, the inverse of a product of at
// most 4 (bounded by the chunked mode's decay domain), so every one of them
// is a plain product per column half.
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
// M <= 64 and N multiples of 4, any K.  fa(m, k) and fb(k, n) return operand
// elements (fp32); fe(m, n, v) consumes each result.  AK: A's memory is
// contiguous along k (else along m); BN: B's memory is contiguous along n
// (else along k) -- consecutive threads then load consecutive addresses.
// The columns are taken 128 at a time; each thread owns two 4x4 output
// tiles.  K-slices of both operands are staged in LDS (rows padded against
// bank conflicts), the next slice loaded into registers while the current
// one is used.  Ends with a barrier, so the next product may read what fe
// wrote.
// ---------------------------------------------------------------------------
constexpr int kGK = 16;
struct __attribute__((aligned(16))) GemmLds {
    float a[kGK][64 + 4];
    float b[kGK][128 + 4];
};

template <bool AK, bool BN, typename FA, typename FB, typename FE>
__device__ __attribute__((always_inline)) inline void gemm(GemmLds& sm, int M, int N, int K, FA fa, FB fb, FE fe)
{
    const int tid = threadIdx.x;
    for (int nb = 0; nb < N; nb += 128) {
        const int NB = N - nb < 128 ? N - nb : 128;
        const int tnc = NB / 4, nsl = (M / 4) * tnc;      // <= 512 tiles
        // staging element u of this thread: A (m, kk), B (kk, n)
        auto a_of = [&](int i, int& m, int& kk) {
            if (AK) { m = i / kGK; kk = i % kGK; } else { kk = i / M; m = i - kk * M; }
        };
        auto b_of = [&](int i, int& kk, int& n) {
            if (BN) { kk = i / NB; n = i - kk * NB; } else { n = i / kGK; kk = i % kGK; }
        };
        float ra[4], rb[8];
        float acc[2][4][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[t][i][j] = 0.f;
        for (int k0 = -kGK; k0 < K; k0 += kGK) {
            if (k0 >= 0) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = tid + u * kThreads;
                    int m, kk;
                    a_of(i, m, kk);
                    if (i < M * kGK) sm.a[kk][m] = ra[u];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = tid + u * kThreads;
                    int kk, n;
                    b_of(i, kk, n);
                    if (i < kGK * NB) sm.b[kk][n] = rb[u];
                }
                __syncthreads();
            }
            const int kn = k0 + kGK;                      // slice to fetch now
            if (kn < K) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = tid + u * kThreads;
                    int m, kk;
                    a_of(i, m, kk);
                    ra[u] = (i < M * kGK && kn + kk < K) ? fa(m, kn + kk) : 0.f;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = tid + u * kThreads;
                    int kk, n;
                    b_of(i, kk, n);
                    rb[u] = (i < kGK * NB && kn + kk < K) ? fb(kn + kk, nb + n) : 0.f;
                }
            }
            if (k0 >= 0) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int slot = tid + t * kThreads;
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
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int slot = tid + t * kThreads;
            if (slot < nsl) {
                const int m0 = 4 * (slot / tnc), n0 = 4 * (slot - (slot / tnc) * tnc);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) fe(m0 + i, nb + n0 + j, acc[t][i][j]);
            }
        }
    }
    __syncthreads();
}

template <typename T> __device__ inline float ldf(const T* p, int64_t i) { return Io<T>::to_f(p[i]); }
template <typename T> __device__ inline void stf(T* p, int64_t i, float x) { p[i] = Io<T>::from_f(x); }

// ---------------------------------------------------------------------------
// launch 3: reverse pass over chunks
//
// One workgroup per (batch, head, slice of VS value columns).  The chunk's
// factors are copied byte for byte from the front of its workspace block
// (Qh, W, Ktil^T, P, Gamma_L: everything before U^T) into an LDS image,
// with the chunk's dO columns behind it; the copy of chunk n-1 is loaded
// into registers (16-byte granules) while chunk n is computed.  The state
// gradient dS [DK][VS] and dDelta [64][VS] stay in LDS in fp32; the two
// products per chunk run on the matrix cores (fp32 accumulation), their
// fragments gathered element by element from the LDS image.
// ---------------------------------------------------------------------------
template <typename Tio, int DK>
struct BwdStateLds {
    static constexpr int ES = (int)sizeof(Tio), KB = Io<Tio>::KB;
    static constexpr WsLayout LY = ws_layout(DK, 0, sizeof(Tio), KB);
    static constexpr int IMG = (int)LY.uwyt;                 // bytes of the factor image
};

template <typename Tio, int DK, int VS>
__global__ __launch_bounds__(kThreads, 1) void k_chunk_state_bwd(BwdStateArgs a)
{
    using SL = BwdStateLds<Tio, DK>;
    constexpr int ES = SL::ES, IMG = SL::IMG;
    constexpr int KPAD = round_up(DK, SL::KB);
    constexpr int GROW = VS * ES / 16;                     // granules of one dO row slice
    constexpr int NG = IMG / 16 + 64 * GROW;                // granules per chunk
    constexpr int NPT = (NG + kThreads - 1) / kThreads;
    constexpr int NCG = VS / 4;                             // column groups
    using IO = Io<Tio>;
    typedef typename IO::frag frag;
    constexpr int EPL = IO::EPL, KB = IO::KB;
    static_assert(IMG % 16 == 0 && VS == 16, "layout: the slice is one 16-column tile");

    __shared__ __attribute__((aligned(16))) char img[IMG + 64 * VS * ES];
    __shared__ __attribute__((aligned(16))) float dS[DK * VS];
    __shared__ __attribute__((aligned(16))) float dD[64 * VS];
    const Tio* P = reinterpret_cast<const Tio*>(img + SL::LY.p);       // [64][64]
    const Tio* Kt = reinterpret_cast<const Tio*>(img + SL::LY.ktt);    // [DK][64]
    const Tio* Qh = reinterpret_cast<const Tio*>(img + SL::LY.qh);     // [64][KPAD]
    const Tio* Wf = reinterpret_cast<const Tio*>(img + SL::LY.wwy);    // [64][KPAD]
    const float* gam = reinterpret_cast<const float*>(img + SL::LY.gaml);
    const Tio* dOs = reinterpret_cast<const Tio*>(img + IMG);          // [64][VS]

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4, wave = tid >> 6;
    const int dv = a.dv;
    f32x4 accD = {0.f, 0.f, 0.f, 0.f};
    // the slices of one head get block ids congruent mod 8 (one XCD, one L2
    // for the head's factors)
    const int64_t nch = a.B * a.H, x = blockIdx.x;
    const int ns = a.nslices;
    int64_t chain;
    int slice;
    if ((nch & 7) == 0) {
        chain = (x / (8 * ns)) * 8 + (x & 7);
        slice = (int)((x >> 3) % ns);
    } else {
        chain = x / ns;
        slice = (int)(x - chain * ns);
    }
    const int j0 = slice * VS;
    const int64_t bb = chain / a.H, hh = chain - bb * a.H;
    const Tio* dO = static_cast<const Tio*>(a.dO);
    // the sequence's tokens, chunk count and first block
    const ChainSpan sp = chain_span(a.plan, a.ncmax, a.B, a.T, a.H, a.nt, bb, hh);
    const int nt = sp.nt;

    f32x4 pre[NPT];
    auto fetch = [&](int n) {
        const char* blk = static_cast<const char*>(a.ws) + (sp.blk0 + n) * a.ws_block;
        const int64_t t0 = (int64_t)n * kChunk;
        const int L = (int)(sp.tlen - t0 < kChunk ? sp.tlen - t0 : kChunk);
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int gi = tid + i * kThreads;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (gi < IMG / 16) {
                x = *reinterpret_cast<const f32x4*>(blk + 16 * gi);
            } else if (gi < NG) {
                const int r = (gi - IMG / 16) / GROW, g = (gi - IMG / 16) % GROW;
                if (r < L)
                    x = *reinterpret_cast<const f32x4*>(
                        dO + ((sp.tok0 + t0 + r) * a.H + hh) * dv + j0 + g * (16 / ES));
            }
            pre[i] = x;
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int gi = tid + i * kThreads;
            if (gi < NG) *reinterpret_cast<f32x4*>(img + 16 * gi) = pre[i];
        }
    };

    for (int i = tid; i < DK * VS; i += kThreads) {
        const int c = i / VS, j = i - c * VS;
        dS[i] = a.dS_T ? a.dS_T[(chain * DK + c) * dv + j0 + j] : 0.f;
    }
    if (nt > 0) fetch(nt - 1);
    for (int n = nt - 1; n >= 0; --n) {
        __syncthreads();                                   // the previous chunk is done with LDS
        stash();
        // the gradient this chunk's exit state receives
        if (a.dSL != nullptr) {
            float* dsl = a.dSL + (sp.blk0 + n) * (int64_t)DK * dv + j0;
            for (int i = tid; i < DK * VS / 4; i += kThreads) {
                const int c = i / NCG, g = i - c * NCG;
                *reinterpret_cast<f32x4*>(dsl + (int64_t)c * dv + 4 * g) = *reinterpret_cast<const f32x4*>(&dS[c * VS + 4 * g]);
            }
        }
        if (a.dSLIo != nullptr) {
            // the same in the I/O dtype
            Tio* dsl = static_cast<Tio*>(a.dSLIo) + (sp.blk0 + n) * (int64_t)DK * dv + j0;
            for (int i = tid; i < DK * VS / 4; i += kThreads) {
                const int c = i / NCG, g = i - c * NCG;
                st_vec4(dsl + (int64_t)c * dv + 4 * g, *reinterpret_cast<const f32x4*>(&dS[c * VS + 4 * g]));
            }
        }
        if (a.dSLT != nullptr) {
            // and transposed, [dv][dk] in the I/O dtype
            Tio* dslT = static_cast<Tio*>(a.dSLT) + (sp.blk0 + n) * (int64_t)DK * dv;
            for (int i = tid; i < DK * VS / 4; i += kThreads) {
                const int j = i / (DK / 4), c4 = 4 * (i - j * (DK / 4));
                const f32x4 x = {dS[c4 * VS + j], dS[(c4 + 1) * VS + j], dS[(c4 + 2) * VS + j], dS[(c4 + 3) * VS + j]};
                st_vec4(dslT + (int64_t)(j0 + j) * DK + c4, x);
            }
        }
        if (n > 0) fetch(n - 1);
        __syncthreads();
        // dDelta = P^T dO + Ktil dS on the matrix cores: wave w owns rows
        // 16w .. 16w+15 (the slice is one 16-column tile); operand fragments are
        // gathered from the LDS image (P and Ktil^T are stored with the
        // contraction index outermost)
        {
#pragma unroll
            for (int kb = 0; kb < 64 / KB; ++kb) {
                frag fa, fb;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const int k = kb * KB + grp * EPL + e;
                    fa[e] = P[k * 64 + 16 * wave + l16];
                    fb[e] = dOs[k * VS + l16];
                }
                accD = IO::mma(accD, fa, fb);
            }
#pragma unroll
            for (int kb = 0; kb < (DK + KB - 1) / KB; ++kb) {
                frag fa, fb;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const int k = kb * KB + grp * EPL + e;
                    fa[e] = k < DK ? Kt[k * 64 + 16 * wave + l16] : IO::from_f(0.f);
                    fb[e] = IO::from_f(k < DK ? dS[k * VS + l16] : 0.f);
                }
                accD = IO::mma(accD, fa, fb);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) dD[(16 * wave + 4 * grp + i) * VS + l16] = accD[i];
            accD = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();
        // dS = Gamma_L dS + Qh^T dO - W^T dDelta: 16-row tiles of dS, one per wave in turn
        for (int tc = wave; tc < DK / 16; tc += 4) {
            f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1;
#pragma unroll
            for (int kb = 0; kb < 64 / KB; ++kb) {
                frag fq, fw, fo, fd;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const int k = kb * KB + grp * EPL + e;
                    fq[e] = Qh[k * KPAD + 16 * tc + l16];
                    fw[e] = Wf[k * KPAD + 16 * tc + l16];
                    fo[e] = dOs[k * VS + l16];
                    fd[e] = IO::from_f(dD[k * VS + l16]);
                }
                a1 = IO::mma(a1, fq, fo);
                a2 = IO::mma(a2, fw, fd);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 16 * tc + 4 * grp + i;
                dS[c * VS + l16] = gam[c] * dS[c * VS + l16] + a1[i] - a2[i];
            }
        }
    }
    __syncthreads();
    if (a.dS0 != nullptr) {
        for (int i = tid; i < DK * VS; i += kThreads) {
            const int c = i / VS, j = i - c * VS;
            a.dS0[(chain * DK + c) * dv + j0 + j] = dS[i];
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
    const int dk = a.dk, dv = a.dv;
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

    for (int64_t ci = blockIdx.x; ci < a.total; ci += gridDim.x) {   // ci: workspace block
        ChunkPos cp;
        if (!chunk_pos(a.plan, a.ncmax, a.B, a.T, a.H, a.nt, ci, cp)) continue;   // past a packed batch's chunks
        const int L = cp.len;
        const int64_t row0 = cp.tok0 * a.H + cp.hh;             // row of the chunk's first token
        const int64_t H = a.H;
        const float* S0 = a.S_chk + ci * (int64_t)dk * dv;      // [dk][dv]
        const float* dSL = a.dSL + ci * (int64_t)dk * dv;

        // ---- G: cumulative log decay (padding tokens have alpha = 1)
        for (int c = tid; c < dk; c += kThreads) {
            float g = 0.f;
            for (int r = 0; r < 64; ++r) {
                if (r < L) g += __logf(fmaxf(ldf(alpha, (row0 + r * H) * dk + c), kAlphaFloor));
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
            KY[i] = kv * __expf(G[((r & ~7) | 3) * dk + c] - g);   // referred to the half's token 3
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

        // ---- A (s < r) and P (s <= r), one 8-column half at a time (rows from
        // the half's first token on; reference token j0 + 3)
        for (int J = 0; J < 8; ++J) {
            const int j0 = 8 * J, jm = j0 + 3;
            gemm<true, false>(gl, 64 - j0, 8, dk,
                 [&](int m, int c) { return ef[(j0 + m) * dk + c] * __expf(G[(j0 + m) * dk + c] - G[jm * dk + c]); },
                 [&](int c, int s) { return KY[(j0 + s) * dk + c]; },
                 [&](int m, int s, float x) { if (s < m) A[(j0 + m) * 64 + j0 + s] = x; });
            gemm<true, false>(gl, 64 - j0, 8, dk,
                 [&](int m, int c) { return qf[(j0 + m) * dk + c] * __expf(G[(j0 + m) * dk + c] - G[jm * dk + c]); },
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
        gemm<true, true>(gl, 64, dv, 64, [&](int m, int s) { return Tm[m * 64 + s]; }, [&](int s, int j) { return u[s * dv + j]; },
             [&](int m, int j, float x) { U[m * dv + j] = x; });
        gemm<true, true>(gl, 64, dk, 64, [&](int m, int s) { return Tm[m * 64 + s]; }, [&](int s, int c) { return Eh[s * dk + c]; },
             [&](int m, int c, float x) { W[m * dk + c] = x; });
        // ---- Delta = U - W S0;  dDelta = P^T dO + Ktil dSL
        gemm<true, true>(gl, 64, dv, dk, [&](int m, int c) { return W[m * dk + c]; },
             [&](int c, int j) { return S0[(int64_t)c * dv + j]; },
             [&](int m, int j, float x) { Dl[m * dv + j] = U[m * dv + j] - x; });
        gemm<false, true>(gl, 64, dv, 64, [&](int m, int s) { return P[s * 64 + m]; },
                          [&](int s, int j) { return dOf[s * dv + j]; }, [&](int m, int j, float x) { dDl[m * dv + j] = x; });
        gemm<true, true>(gl, 64, dv, dk, [&](int m, int c) { return Kt[m * dk + c]; },
                         [&](int c, int j) { return dSL[(int64_t)c * dv + j]; },
                         [&](int m, int j, float x) { dDl[m * dv + j] += x; });
        // ---- dQh, dP, dKtil, dW, du (-> dw, dv), dGamma_L
        gemm<true, false>(gl, 64, dk, dv, [&](int m, int j) { return dOf[m * dv + j]; },
             [&](int j, int c) { return S0[(int64_t)c * dv + j]; }, [&](int m, int c, float x) { dQh[m * dk + c] = x; });
        gemm<true, false>(gl, 64, 64, dv, [&](int m, int j) { return dOf[m * dv + j]; }, [&](int j, int s) { return Dl[s * dv + j]; },
             [&](int m, int s, float x) { dP[m * 64 + s] = s <= m ? x : 0.f; });
        gemm<true, false>(gl, 64, dk, dv, [&](int m, int j) { return Dl[m * dv + j]; },
             [&](int j, int c) { return dSL[(int64_t)c * dv + j]; }, [&](int m, int c, float x) { dKt[m * dk + c] = x; });
        gemm<true, false>(gl, 64, dk, dv, [&](int m, int j) { return dDl[m * dv + j]; },
             [&](int j, int c) { return S0[(int64_t)c * dv + j]; }, [&](int m, int c, float x) { dW[m * dk + c] = -x; });
        gemm<false, true>(gl, 64, dv, 64, [&](int m, int s) { return Tm[s * 64 + m]; }, [&](int s, int j) { return dDl[s * dv + j]; },
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
        gemm<true, false>(gl, 64, 64, dv + dk,
             [&](int m, int kk) { return kk < dv ? dDl[m * dv + kk] : dW[m * dk + kk - dv]; },
             [&](int kk, int s) { return kk < dv ? u[s * dv + kk] : Eh[s * dk + kk - dv]; },
             [&](int m, int s, float x) { dT[m * 64 + s] = x; });
        gemm<false, true>(gl, 64, dk, 64, [&](int m, int s) { return Tm[s * 64 + m]; }, [&](int s, int c) { return dW[s * dk + c]; },
             [&](int m, int c, float x) { dEh[m * dk + c] = x; });
        gemm<false, true>(gl, 64, 64, 64, [&](int m, int s) { return Tm[s * 64 + m]; }, [&](int s, int j) { return dT[s * 64 + j]; },
             [&](int m, int j, float x) { tmp[m * 64 + j] = x; });
        gemm<true, false>(gl, 64, 64, 64, [&](int m, int j) { return tmp[m * 64 + j]; }, [&](int j, int s) { return Tm[s * 64 + j]; },
             [&](int m, int s, float x) { dA[m * 64 + s] = s < m ? -x : 0.f; });

        // ---- through A and P: row side (rows r >= j0 of column half J) and
        // column side (columns s of half J), reference token j0 + 3
        for (int J = 0; J < 8; ++J) {
            const int j0 = 8 * J, jm = j0 + 3;
            gemm<true, true>(gl, 64 - j0, dk, 8, [&](int m, int s) { return dA[(j0 + m) * 64 + j0 + s]; },
                 [&](int s, int c) { return KY[(j0 + s) * dk + c]; },
                 [&](int m, int c, float x) {
                     const int r = j0 + m;
                     deA[r * dk + c] += x * __expf(G[r * dk + c] - G[jm * dk + c]);
                 });
            gemm<true, true>(gl, 64 - j0, dk, 8, [&](int m, int s) { return m == s ? 0.f : dP[(j0 + m) * 64 + j0 + s]; },
                 [&](int s, int c) { return KY[(j0 + s) * dk + c]; },
                 [&](int m, int c, float x) {
                     const int r = j0 + m;
                     dqP[r * dk + c] += x * __expf(G[r * dk + c] - G[jm * dk + c]);
                 });
            gemm<false, true>(gl, 8, dk, 64 - j0, [&](int m, int rr) { return dA[(j0 + rr) * 64 + j0 + m]; },
                 [&](int rr, int c) {
                     const int r = j0 + rr;
                     return ef[r * dk + c] * __expf(G[r * dk + c] - G[jm * dk + c]);
                 },
                 [&](int m, int c, float x) {
                     const int s = j0 + m;
                     dkA[s * dk + c] += x * __expf(G[jm * dk + c] - G[s * dk + c]);
                 });
            gemm<false, true>(gl, 8, dk, 64 - j0, [&](int m, int rr) { return m == rr ? 0.f : dP[(j0 + rr) * 64 + j0 + m]; },
                 [&](int rr, int c) {
                     const int r = j0 + rr;
                     return qf[r * dk + c] * __expf(G[r * dk + c] - G[jm * dk + c]);
                 },
                 [&](int m, int c, float x) {
                     const int s = j0 + m;
                     dkP[s * dk + c] += x * __expf(G[jm * dk + c] - G[s * dk + c]);
                 });
        }

        // ---- gradients of q, k, b and of G (dG kept in deA's place; P's
        // diagonal, left out of dqP and dkP, added to dq and dk here)
        for (int i = tid; i < KA; i += kThreads) {
            const int r = i / dk, c = i - r * dk;
            const float g = G[i], gam = __expf(g);
            const float de = gam * dEh[i] + deA[i];
            const float kv = kf[i], pd = dP[r * 64 + r];
            const bool ok = r < L;
            const int64_t o = (row0 + r * H) * dk + c;
            const float bv = ok ? ldf(bg, o) : 0.f;
            const float dG = dQh[i] * Qh[i] + dEh[i] * Eh[i] + ef[i] * deA[i] + qf[i] * dqP[i] -
                             kv * (dkA[i] + dkP[i]);
            if (ok) {
                stf(dq, o, gam * dQh[i] + dqP[i] + pd * kv);
                stf(dk_out, o, __expf(G[63 * dk + c] - g) * dKt[i] + dkA[i] + dkP[i] + pd * qf[i] + de * bv);
                stf(db, o, de * kv);
            }
            deA[i] = dG;
        }
        __syncthreads();
        // dlog(alpha_t): the reverse sum of dG from t on, Gamma_L's uses, and
        // the forward sum of Ktil's terms over the tokens before t
        for (int c = tid; c < dk; c += kThreads) {
            float pre = 0.f;
            for (int r = 0; r < 64; ++r) {
                const float x = dKt[r * dk + c] * Kt[r * dk + c];
                dKt[r * dk + c] = pre;
                pre += x;
            }
            float acc = dGamL[c] * __expf(G[63 * dk + c]);
            for (int r = 63; r >= 0; --r) {
                acc += deA[r * dk + c];
                if (r < L) {
                    const int64_t o = (row0 + r * H) * dk + c;
                    {   // a decay below the floor was raised to it: its gradient is 0
                        const float al = ldf(alpha, o);
                        stf(dalpha, o, al < kAlphaFloor ? 0.f : (acc + dKt[r * dk + c]) / al);
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#ifndef GDN2_GRAD_BLOCKS
#define GDN2_GRAD_BLOCKS 1024
#endif
int64_t grad_blocks(int64_t total) { return total < GDN2_GRAD_BLOCKS ? total : GDN2_GRAD_BLOCKS; }

int64_t chunk_grad_scratch_bytes(int dk, int dv, int64_t total)
{
    return grad_blocks(total) * grad_scratch_floats(dk, dv) * 4;
}

template <typename Tio, int DK>
static hipError_t state_bwd_dk(const BwdStateArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)(a.B * a.H * (int64_t)a.nslices));
    if (a.vs != 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_chunk_state_bwd<Tio, DK, 16>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename Tio>
static hipError_t state_bwd_t(const BwdStateArgs& a, hipStream_t s)
{
    switch (a.dk) {
        case 16: return state_bwd_dk<Tio, 16>(a, s);
        case 32: return state_bwd_dk<Tio, 32>(a, s);
        case 64: return state_bwd_dk<Tio, 64>(a, s);
        case 128: return state_bwd_dk<Tio, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

// value-slice width of the reverse state pass
// (16 columns: twice the workgroups of 32 and half the serial work per chunk)
int state_bwd_slice(int dv) { return dv % 16 == 0 ? 16 : 0; }

hipError_t launch_chunk_state_bwd(const BwdStateArgs& a, bool bf16, hipStream_t s)
{
    return bf16 ? state_bwd_t<__bf16>(a, s) : state_bwd_t<float>(a, s);
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
