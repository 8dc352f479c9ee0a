// Chunked forward of the GDN-2 token mixer on gfx950: the two kernels behind
// gdn2_chunk_fwd.
//
// The pages (burn-gdn2 0.1.9 README, intro and "Architecture") name a chunked
// WY decomposition with chunk size 64 ("Configuration") as the training-mode
// forward but give no formulas.  The form used here follows from the
// per-token recurrence S_t = (I - k (b*k)^T) diag(alpha) S + k (w*v)^T,
// o_t = q^T S_t.  For one chunk entering with state S (positions r, s):
//
//   Gamma_r = prod_{j<=r} alpha_j (per key channel), e_r = b_r * k_r, u_r = w_r * v_r
//   A[r][s] = sum_c e_r[c] k_s[c] Gamma_r[c]/Gamma_s[c]   (s <  r)
//   P[r][s] = sum_c q_r[c] k_s[c] Gamma_r[c]/Gamma_s[c]   (s <= r)
//   T = (I + A)^{-1},  W = T (Gamma * e),  U = T u
//   Delta = U - W S,   O = (Gamma * q) S + P Delta
//   S'    = diag(Gamma_L) S + Ktil^T Delta,  Ktil_s = k_s Gamma_L / Gamma_s
//
// k_chunk_prep (one workgroup per (batch, head, chunk), all in parallel)
// builds every S-independent factor and stores it in the workspace;
// k_chunk_state (one workgroup per (batch, head, value slice)) runs the
// chunks in order with the fp32 state held in matrix-core accumulators.
//
// Decay ratios inside matrix products.  Gamma_r/Gamma_s is split over the four
// 16-token blocks of the chunk: with g_r the running product of alpha from the
// start of r's block (so g <= 1) and Z_K the product over block K,
//   same block:   Gamma_r/Gamma_s = g_r * (1/g_s)
//   block I > J:  Gamma_r/Gamma_s = g_r * (1/g_s) * prod_{K=J}^{I-1} Z_K
// so one row-side operand (e*g, q*g) and one column-side operand (k/g) serve
// every block pair; the off-diagonal factor is applied per channel to the
// column operand on load.  Only 1/g_s can exceed 1, by at most the inverse
// decay of 16 tokens.  No exp/log is evaluated: all factors are running
// products of alpha.
#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"
#include "gdn2_layout.hpp"

namespace gdn2 {

__host__ __device__ constexpr int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr int align16(int x) { return (x + 15) & ~15; }

// ---------------------------------------------------------------------------
// k_chunk_prep
// ---------------------------------------------------------------------------
template <typename Tio, int DK>
struct PrepSmem {
    static constexpr int EPL = Io<Tio>::EPL, KB = Io<Tio>::KB, ES = (int)sizeof(Tio);
    static constexpr int KPAD = round_up(DK, KB);
    static constexpr int RS = KPAD + EPL;   // row stride of [64][KPAD] operand arrays (elements)
    static constexpr int TS = 64 + EPL;     // row stride of [*][64] operand arrays (elements)
    static constexpr int FS = 68;           // row stride of fp32 64x64 matrices
    static constexpr int SZ_X = 64 * RS * ES;
    static constexpr int SZ_F64 = 64 * FS * 4;
    static constexpr int SZ_T = 64 * TS * ES;
    static constexpr int SZ_BSC = 16 * 48 * 4;
    // R0: Xe -> A32 -> UT;  R1: Xq -> T32;  R2: Yd -> (Tm, Bsc);  R3: EhT
    static constexpr int R0 = align16(imax(imax(SZ_X, SZ_F64), SZ_T));
    static constexpr int R1 = align16(imax(SZ_X, SZ_F64));
    static constexpr int R2 = align16(imax(SZ_X, SZ_T + SZ_BSC));
    static constexpr int R3 = align16(KPAD * TS * ES);
    static constexpr int O1 = R0, O2 = O1 + R1, O3 = O2 + R2, OZ = O3 + R3;
    static constexpr int OF = OZ + 4 * DK * 4;          // Zs [4][DK]
    static constexpr int BYTES = OF + 6 * KPAD * 4;     // Fs [6][KPAD]
};

// block pairs (I >= J) of the 64x64 lower triangle, diagonal first; the
// off-diagonal order matches the rows of the factor table Fs.
// (packed 2 bits per entry so that a wave-dependent index needs no table in memory)
__host__ __device__ constexpr unsigned pack2(const int (&v)[10], int n) {
    unsigned r = 0;
    for (int i = 0; i < n; ++i) r |= unsigned(v[i]) << (2 * i);
    return r;
}
constexpr int kPairIv[10] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3};
constexpr int kPairJv[10] = {0, 1, 2, 3, 0, 1, 2, 0, 1, 0};
constexpr int kUpperIv[10] = {0, 1, 2, 0, 1, 0, 0, 0, 0, 0};
constexpr int kUpperJv[10] = {1, 2, 3, 2, 3, 3, 0, 0, 0, 0};
constexpr unsigned kPairI = pack2(kPairIv, 10), kPairJ = pack2(kPairJv, 10);
constexpr unsigned kUpperI = pack2(kUpperIv, 6), kUpperJ = pack2(kUpperJv, 6);
__device__ inline int unpack2(unsigned p, int i) { return (int)((p >> (2 * i)) & 3u); }

// NUI = (token, 4-column) value items per thread: 64 * dv / 4 <= 256 * NUI
template <typename Tio, int DK, int NUI>
__global__ __launch_bounds__(kThreads, 2) void k_chunk_prep(PrepArgs a)
{
    using IO = Io<Tio>;
    using SM = PrepSmem<Tio, DK>;
    constexpr int EPL = SM::EPL, KB = SM::KB, KPAD = SM::KPAD, RS = SM::RS, TS = SM::TS, FS = SM::FS;
    constexpr WsLayout LY = ws_layout(DK, 0, sizeof(Tio), KB);

    __shared__ __attribute__((aligned(16))) char smem[SM::BYTES];
    Tio* Xe = reinterpret_cast<Tio*>(smem);
    float* A32 = reinterpret_cast<float*>(smem);
    Tio* UT = reinterpret_cast<Tio*>(smem);
    Tio* Xq = reinterpret_cast<Tio*>(smem + SM::O1);
    float* T32 = reinterpret_cast<float*>(smem + SM::O1);
    Tio* Yd = reinterpret_cast<Tio*>(smem + SM::O2);
    Tio* Tm = reinterpret_cast<Tio*>(smem + SM::O2);
    float* Bsc = reinterpret_cast<float*>(smem + SM::O2 + SM::SZ_T);
    Tio* EhT = reinterpret_cast<Tio*>(smem + SM::O3);
    float* Zs = reinterpret_cast<float*>(smem + SM::OZ);
    float* Fs = reinterpret_cast<float*>(smem + SM::OF);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int64_t chi = blockIdx.x;
    const int64_t chain = chi / a.nt;
    const int n = (int)(chi - chain * a.nt);
    const int64_t bb = chain / a.H, hh = chain - bb * a.H;
    const int64_t t0 = (int64_t)n * kChunk;
    const int L = (int)((a.T - t0) < kChunk ? (a.T - t0) : kChunk);
    const int64_t row0 = (bb * a.T + t0) * a.H + hh;    // row of token t0 in [B,T,H,*]
    const int64_t H = a.H;
    const Tio* q = static_cast<const Tio*>(a.q);
    const Tio* k = static_cast<const Tio*>(a.k);
    const Tio* v = static_cast<const Tio*>(a.v);
    char* blk = static_cast<char*>(a.ws) + chi * a.ws_block;
    Tio* qh_out = reinterpret_cast<Tio*>(blk + LY.qh);
    Tio* wwy_out = reinterpret_cast<Tio*>(blk + LY.wwy);
    Tio* ktt_out = reinterpret_cast<Tio*>(blk + LY.ktt);
    Tio* p_out = reinterpret_cast<Tio*>(blk + LY.p);
    float* gaml_out = reinterpret_cast<float*>(blk + LY.gaml);
    Tio* uwyt_out = reinterpret_cast<Tio*>(blk + LY.uwyt);

    typedef typename IO::frag frag;
    typedef typename IO::pair pair2;

    // ---- 0. every global load of the kernel, before any global store --------
    // One vector-memory counter tracks loads and stores alike, so a load
    // issued after a store would also wait for that store to complete.  Loads
    // are unconditional (rows past the sequence end are clamped to its last
    // row and replaced by identity tokens afterwards): a load under a branch
    // would be waited for at the join.  16-byte accesses keep the count of
    // loads per lane under the 63 the counter can track.
    // Key-axis item = (4 channels c0..c0+3, 8-token group rg); block p = rg/2.
    constexpr int NQ = DK / 4;
    const bool kact = tid < 2 * DK;
    const int cq = tid % NQ, rg = (tid / NQ) & 7, p = rg >> 1, half = rg & 1, c0 = 4 * cq;
    f32x4 al[8], bt[8];
    typename IO::vec4 kk[8], qq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 8 * rg + i;
        const int64_t off = (row0 + (r < L ? r : L - 1) * H) * DK + c0;
        al[i] = *reinterpret_cast<const f32x4*>(a.alpha + off);
        bt[i] = *reinterpret_cast<const f32x4*>(a.b + off);
        kk[i] = *reinterpret_cast<const typename IO::vec4*>(k + off);
        qq[i] = *reinterpret_cast<const typename IO::vec4*>(q + off);
    }
    // value-axis item = (token s, 4 columns): u = w * v
    constexpr int NVQ_MAX = NUI;
    f32x4 wr[NVQ_MAX];
    typename IO::vec4 vr[NVQ_MAX];
    const int nvq = a.dv / 4;
#pragma unroll
    for (int m = 0; m < NVQ_MAX; ++m) {
        const int u = tid + m * kThreads;
        const int jq = u % nvq, s = u / nvq;
        const int64_t off = (row0 + (s < L ? s : L - 1) * H) * a.dv + 4 * jq;
        wr[m] = *reinterpret_cast<const f32x4*>(a.w + off);
        vr[m] = *reinterpret_cast<const typename IO::vec4*>(v + off);
    }
    f32x4 uu[NVQ_MAX];
#pragma unroll
    for (int m = 0; m < NVQ_MAX; ++m) {
        const int s = (tid + m * kThreads) / nvq;
        uu[m] = (s < L && s < 64) ? wr[m] * IO::unpack4(vr[m]) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (!(kact && 8 * rg + i < L)) {
            al[i] = f32x4{1.f, 1.f, 1.f, 1.f};
            bt[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            kk[i] = IO::pack4(f32x4{0.f, 0.f, 0.f, 0.f});
            qq[i] = kk[i];
        }
    }

    // ---- 1a. running decay products inside each 16-token block -------------
    // g[i] = prod of alpha from the start of the 16-token block to row i; the
    // second 8-token half multiplies in the first half's total (lane +- NQ).
    f32x4 g[8];
    f32x4 zblk;
    {
        f32x4 run = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            run *= al[i];
            g[i] = run;
        }
        f32x4 other;
#pragma unroll
        for (int e = 0; e < 4; ++e) other[e] = __shfl_xor(run[e], NQ, 64);
        if (half) {
#pragma unroll
            for (int i = 0; i < 8; ++i) g[i] *= other;
        }
        zblk = run * other;
        if (kact && half == 0) *reinterpret_cast<f32x4*>(Zs + p * DK + c0) = zblk;
    }
    if constexpr (KPAD > DK) {   // zero the K padding of the operand arrays
        for (int e = tid; e < 64 * (KPAD - DK); e += kThreads) {
            const int r = e / (KPAD - DK), c = DK + e % (KPAD - DK);
            Xe[r * RS + c] = IO::from_f(0.f);
            Xq[r * RS + c] = IO::from_f(0.f);
            Yd[r * RS + c] = IO::from_f(0.f);
            EhT[c * TS + r] = IO::from_f(0.f);
            qh_out[r * KPAD + c] = IO::from_f(0.f);
            wwy_out[r * KPAD + c] = IO::from_f(0.f);
        }
        for (int e = tid; e < 6 * (KPAD - DK); e += kThreads)
            Fs[(e / (KPAD - DK)) * KPAD + DK + e % (KPAD - DK)] = 0.f;
    }
    __syncthreads();

    // ---- 1b. block factors, decay-scaled operands ---------------------------
    if (kact) {
        f32x4 z[4];
#pragma unroll
        for (int K = 0; K < 4; ++K) z[K] = *reinterpret_cast<const f32x4*>(Zs + K * DK + c0);
        if (rg == 0) {
            *reinterpret_cast<f32x4*>(Fs + 0 * KPAD + c0) = z[0];                 // pair (1,0)
            *reinterpret_cast<f32x4*>(Fs + 1 * KPAD + c0) = z[1];                 // pair (2,1)
            *reinterpret_cast<f32x4*>(Fs + 2 * KPAD + c0) = z[2];                 // pair (3,2)
            *reinterpret_cast<f32x4*>(Fs + 3 * KPAD + c0) = z[0] * z[1];          // pair (2,0)
            *reinterpret_cast<f32x4*>(Fs + 4 * KPAD + c0) = z[1] * z[2];          // pair (3,1)
            *reinterpret_cast<f32x4*>(Fs + 5 * KPAD + c0) = z[0] * z[1] * z[2];   // pair (3,0)
            *reinterpret_cast<f32x4*>(gaml_out + c0) = z[0] * z[1] * z[2] * z[3];
        }
        f32x4 pre = {1.f, 1.f, 1.f, 1.f}, post = pre;
#pragma unroll
        for (int K = 0; K < 4; ++K) {
            if (K < p) pre *= z[K];
            if (K > p) post *= z[K];
        }
        Tio eh[4][8], kt[4][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * rg + i;
            const f32x4 kv = IO::unpack4(kk[i]), qv = IO::unpack4(qq[i]);
            const f32x4 ig = {fast_rcp(g[i][0]), fast_rcp(g[i][1]), fast_rcp(g[i][2]), fast_rcp(g[i][3])};
            const f32x4 xe = bt[i] * kv * g[i], xq = qv * g[i];
            st_vec4(Xe + r * RS + c0, xe);
            st_vec4(Xq + r * RS + c0, xq);
            st_vec4(Yd + r * RS + c0, kv * ig);
            st_vec4(qh_out + r * KPAD + c0, xq * pre);
            const f32x4 ehv = xe * pre, ktv = kv * (zblk * ig) * post;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                eh[e][i] = IO::from_f(ehv[e]);
                kt[e][i] = IO::from_f(ktv[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int i = 0; i < 8; i += EPL) {
                frag f0, f1;
#pragma unroll
                for (int e2 = 0; e2 < EPL; ++e2) {
                    f0[e2] = eh[e][i + e2];
                    f1[e2] = kt[e][i + e2];
                }
                *reinterpret_cast<frag*>(EhT + (c0 + e) * TS + 8 * rg + i) = f0;
                *reinterpret_cast<frag*>(ktt_out + (c0 + e) * 64 + 8 * rg + i) = f1;
            }
        }
    }
    __syncthreads();

    // ---- 2. A^T and P^T tiles on the matrix cores ---------------------------
    // tile (J, I): rows s of block J, columns r of block I,
    // D[s][r] = sum_c Y[s][c] (f_IJ[c]) X[r][c]
    f32x4 accA[3], accP[3];
#pragma unroll
    for (int pi = 0; pi < 3; ++pi) {
        accA[pi] = f32x4{0.f, 0.f, 0.f, 0.f};
        accP[pi] = accA[pi];
        const int pr = wave + 4 * pi;
        if (pr < 10) {
            const int I = unpack2(kPairI, pr), J = unpack2(kPairJ, pr);
#pragma unroll
            for (int kb = 0; kb < KPAD / KB; ++kb) {
                const int ko = kb * KB + grp * EPL;
                typename IO::frag y = ld_frag(Yd + (16 * J + l16) * RS + ko);
                if (pr >= 4) y = IO::scale(y, Fs + (pr - 4) * KPAD + ko);
                const typename IO::frag xe = ld_frag(Xe + (16 * I + l16) * RS + ko);
                const typename IO::frag xq = ld_frag(Xq + (16 * I + l16) * RS + ko);
                accA[pi] = IO::mma(accA[pi], y, xe);
                accP[pi] = IO::mma(accP[pi], y, xq);
            }
        }
    }
    __syncthreads();   // every read of Xe/Xq/Yd is done; A32 may overwrite Xe
#pragma unroll
    for (int pi = 0; pi < 3; ++pi) {
        const int pr = wave + 4 * pi;
        if (pr < 10) {
            const int I = unpack2(kPairI, pr), J = unpack2(kPairJ, pr);
            const int r = 16 * I + l16;
            f32x4 av = accA[pi], pv = accP[pi];
            if (I == J) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = 4 * grp + i;
                    if (s >= l16) av[i] = 0.f;
                    if (s > l16) pv[i] = 0.f;
                }
            }
            *reinterpret_cast<f32x4*>(A32 + r * FS + 16 * J + 4 * grp) = av;
            st_vec4(p_out + r * 64 + 16 * J + 4 * grp, pv);
        }
    }
    for (int u = wave; u < 6; u += 4) {   // P is zero above the block diagonal
        const int r = 16 * unpack2(kUpperI, u) + l16;
        st_vec4(p_out + r * 64 + 16 * unpack2(kUpperJ, u) + 4 * grp, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    __syncthreads();

    // ---- 3. T = (I + A)^{-1}, fp32, blocked forward substitution -------------
    if (wave == 0) {
        // diagonal 16x16 blocks: lane = (block I, column j)
        const int I = lane >> 4, j = lane & 15;
        const float* Ab = A32 + (16 * I) * FS + 16 * I;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int sp = 0; sp < r; ++sp) s -= Ab[r * FS + sp] * x[sp];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) T32[(16 * I + r) * FS + 16 * I + j] = x[r];
    } else {
        // blocks above the diagonal are zero
        for (int e = tid - 64; e < 6 * 256; e += kThreads - 64) {
            const int u = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
            T32[(16 * unpack2(kUpperI, u) + rr) * FS + 16 * unpack2(kUpperJ, u) + cc] = 0.f;
        }
    }
    __syncthreads();
#pragma unroll
    for (int I = 1; I < 4; ++I) {
        const int ncol = 16 * I;
        // Bsc = A[block I rows][0:16I] * T[0:16I][0:16I]
        for (int e = tid; e < 16 * ncol; e += kThreads) {
            const int rr = e / ncol, cc = e - rr * ncol;
            const float* arow = A32 + (16 * I + rr) * FS;
            float s = 0.f;
#pragma unroll
            for (int sp = 0; sp < ncol; ++sp) s += arow[sp] * T32[sp * FS + cc];
            Bsc[rr * 48 + cc] = s;
        }
        __syncthreads();
        // T[block I rows][0:16I] = -T_II * Bsc
        for (int e = tid; e < 16 * ncol; e += kThreads) {
            const int rr = e / ncol, cc = e - rr * ncol;
            const float* trow = T32 + (16 * I + rr) * FS + 16 * I;
            float s = 0.f;
#pragma unroll
            for (int sp = 0; sp < 16; ++sp) s += trow[sp] * Bsc[sp * 48 + cc];
            T32[(16 * I + rr) * FS + cc] = -s;
        }
        __syncthreads();
    }
    for (int e = tid; e < 64 * 64; e += kThreads) {
        const int r = e >> 6, s = e & 63;
        Tm[r * TS + s] = IO::from_f(s <= r ? T32[r * FS + s] : 0.f);
    }
    __syncthreads();

    // ---- 4. W^T = (Gamma e)^T T^T : tile (c-block, r-block = wave) ----------
    typename IO::frag tf[64 / KB];
#pragma unroll
    for (int kb = 0; kb < 64 / KB; ++kb) tf[kb] = ld_frag(Tm + (16 * wave + l16) * TS + kb * KB + grp * EPL);
#pragma unroll
    for (int ct = 0; ct < DK / 16; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 64 / KB; ++kb) {
            if (kb * KB <= 16 * wave + 15) {
                const typename IO::frag fe = ld_frag(EhT + (16 * ct + l16) * TS + kb * KB + grp * EPL);
                acc = IO::mma(acc, fe, tf[kb]);
            }
        }
        // acc[i] = W[r = 16*wave + l16][c = 16*ct + 4*grp + i]
        st_vec4(wwy_out + (16 * wave + l16) * KPAD + 16 * ct + 4 * grp, acc);
    }

    // ---- 5. U = T (w * v), stored transposed, in column blocks of 64 --------
    for (int j0 = 0; j0 < a.dv; j0 += 64) {
        const int nj = (a.dv - j0) < 64 ? (a.dv - j0) : 64;
#pragma unroll
        for (int m = 0; m < NVQ_MAX; ++m) {
            const int u = tid + m * kThreads;
            const int j = 4 * (u % nvq), s = u / nvq;
            if (s < 64 && j >= j0 && j < j0 + nj) {
#pragma unroll
                for (int e = 0; e < 4; ++e) UT[(j - j0 + e) * TS + s] = IO::from_f(uu[m][e]);
            }
        }
        __syncthreads();
        for (int jt = 0; jt < nj / 16; ++jt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 64 / KB; ++kb) {
                if (kb * KB <= 16 * wave + 15) {
                    const frag fu = ld_frag(UT + (16 * jt + l16) * TS + kb * KB + grp * EPL);
                    acc = IO::mma(acc, tf[kb], fu);
                }
            }
            // acc[i] = U[r = 16*wave + 4*grp + i][j = j0 + 16*jt + l16]
            st_vec4(uwyt_out + (int64_t)(j0 + 16 * jt + l16) * 64 + 16 * wave + 4 * grp, acc);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// k_chunk_state
// ---------------------------------------------------------------------------
// Workgroup = (batch, head, value slice of VS columns).  The slice of S
// (DK x VS, fp32) lives in accumulators: wave w owns row tiles
// [w*SPW, (w+1)*SPW).  Per chunk:
//   X_W = W S, X_Q = Qh S        (wave w: rows of token block w)
//   Delta = U - X_W   -> LDS (transposed, I/O dtype)
//   O = X_Q + P Delta -> o
//   S = diag(Gamma_L) S + Ktil^T Delta -> LDS copy of S (I/O dtype) for the next chunk
// The slices of one head are mapped to one XCD (block id = xcd + 8*k) so that
// the shared workspace blocks are read through a single L2.
template <typename Tio, int DK, int VS>
__global__ __launch_bounds__(kThreads) void k_chunk_state(StateArgs a)
{
    using IO = Io<Tio>;
    constexpr int EPL = IO::EPL, KB = IO::KB;
    constexpr int KPAD = round_up(DK, KB);
    constexpr int NCT = VS / 16;
    constexpr int SRT = DK / 16;
    constexpr int SPW = (SRT + 3) / 4;
    constexpr int SRS = KPAD + EPL;
    constexpr int DTS = 64 + EPL;
    constexpr int NKX = KPAD / KB;
    constexpr int NKT = 64 / KB;
    constexpr WsLayout LY = ws_layout(DK, 0, sizeof(Tio), KB);

    __shared__ __attribute__((aligned(16))) Tio SbT[2][VS * SRS];
    __shared__ __attribute__((aligned(16))) Tio DT[2][VS * DTS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int64_t nch = a.B * a.H;
    const int ns = a.nslices;
    const int64_t x = blockIdx.x;
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
    const int dv = a.dv;
    Tio* o = static_cast<Tio*>(a.o);

    f32x4 accS[SPW][NCT];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int rt = wave * SPW + i;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            if (a.S0 != nullptr && rt < SRT) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s[e] = a.S0[(chain * DK + 16 * rt + 4 * grp + e) * dv + j0 + 16 * ct + l16];
            }
            accS[i][ct] = s;
        }
    }
    if constexpr (KPAD > DK) {
        for (int e = tid; e < 2 * VS * (KPAD - DK); e += kThreads) {
            const int bf = e / (VS * (KPAD - DK)), rem = e % (VS * (KPAD - DK));
            SbT[bf][(rem / (KPAD - DK)) * SRS + DK + rem % (KPAD - DK)] = IO::from_f(0.f);
        }
    }
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int rt = wave * SPW + i;
        if (rt < SRT) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) st_vec4(&SbT[0][(16 * ct + l16) * SRS + 16 * rt + 4 * grp], accS[i][ct]);
        }
    }
    __syncthreads();

    // operands of one chunk, loaded one chunk ahead (registers)
    typedef typename IO::frag frag;
    struct Ops {
        frag w[NKX], q[NKX], p[NKT], k[SPW][NKT];
        typename IO::vec4 u[NCT];
        f32x4 gl[SPW];
    };
    auto load_ops = [&](int n, Ops& op) {
        const char* blk = static_cast<const char*>(a.ws) + (chain * a.nt + n) * a.ws_block;
        const Tio* Qh = reinterpret_cast<const Tio*>(blk + LY.qh);
        const Tio* Ww = reinterpret_cast<const Tio*>(blk + LY.wwy);
        const Tio* Kt = reinterpret_cast<const Tio*>(blk + LY.ktt);
        const Tio* Pm = reinterpret_cast<const Tio*>(blk + LY.p);
        const float* Gl = reinterpret_cast<const float*>(blk + LY.gaml);
        const Tio* Ut = reinterpret_cast<const Tio*>(blk + LY.uwyt);
#pragma unroll
        for (int kb = 0; kb < NKX; ++kb) {
            op.w[kb] = ld_frag(Ww + (16 * wave + l16) * KPAD + kb * KB + grp * EPL);
            op.q[kb] = ld_frag(Qh + (16 * wave + l16) * KPAD + kb * KB + grp * EPL);
        }
        // unconditional loads (rows of idle tiles clamped into range) keep the
        // compiler from waiting at branch joins
#pragma unroll
        for (int kb = 0; kb < NKT; ++kb) {
            op.p[kb] = ld_frag(Pm + (16 * wave + l16) * 64 + kb * KB + grp * EPL);
#pragma unroll
            for (int i = 0; i < SPW; ++i) {
                const int rt = (wave * SPW + i) < SRT ? (wave * SPW + i) : SRT - 1;
                op.k[i][kb] = ld_frag(Kt + (16 * rt + l16) * 64 + kb * KB + grp * EPL);
            }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            op.u[ct] = *reinterpret_cast<const typename IO::vec4*>(Ut + (int64_t)(j0 + 16 * ct + l16) * 64 + 16 * wave + 4 * grp);
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int rt = (wave * SPW + i) < SRT ? (wave * SPW + i) : SRT - 1;
            op.gl[i] = *reinterpret_cast<const f32x4*>(Gl + 16 * rt + 4 * grp);
        }
    };

    // one chunk: prefetch chunk n+1 into `nx`, compute chunk n from `cu`
    auto step = [&](int n, const Ops& cu, Ops& nx) {
        // unconditional (the last chunk reloads itself): a prefetch under a
        // branch makes the compiler drain every outstanding access first
        load_ops(n + 1 < a.nt ? n + 1 : n, nx);
        const Tio* Sb = SbT[n & 1];
        Tio* Dt = DT[n & 1];

        // X_W, X_Q for token block `wave`
        f32x4 accW[NCT], accQ[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            accW[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            accQ[ct] = accW[ct];
        }
#pragma unroll
        for (int kb = 0; kb < NKX; ++kb) {
            const int ko = kb * KB + grp * EPL;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const frag fs = ld_frag(Sb + (16 * ct + l16) * SRS + ko);
                accW[ct] = IO::mma(accW[ct], cu.w[kb], fs);
                accQ[ct] = IO::mma(accQ[ct], cu.q[kb], fs);
            }
        }
        // Delta = U - X_W (rows 16*wave + 4*grp + i, column 16*ct + l16)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            st_vec4(Dt + (16 * ct + l16) * DTS + 16 * wave + 4 * grp, IO::unpack4(cu.u[ct]) - accW[ct]);
        __syncthreads();

        // O = X_Q + P Delta
#pragma unroll
        for (int kb = 0; kb < NKT; ++kb) {
            if (kb * KB <= 16 * wave + 15) {
                const int ko = kb * KB + grp * EPL;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const frag fd = ld_frag(Dt + (16 * ct + l16) * DTS + ko);
                    accQ[ct] = IO::mma(accQ[ct], cu.p[kb], fd);
                }
            }
        }

        // S = diag(Gamma_L) S + Ktil^T Delta
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int rt = wave * SPW + i;
            if (rt < SRT) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) accS[i][ct] *= cu.gl[i];
#pragma unroll
                for (int kb = 0; kb < NKT; ++kb) {
                    const int ko = kb * KB + grp * EPL;
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        const frag fd = ld_frag(Dt + (16 * ct + l16) * DTS + ko);
                        accS[i][ct] = IO::mma(accS[i][ct], cu.k[i][kb], fd);
                    }
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    st_vec4(&SbT[(n + 1) & 1][(16 * ct + l16) * SRS + 16 * rt + 4 * grp], accS[i][ct]);
            }
        }
        // o rows of token block `wave` (after the next chunk's loads were issued)
        {
            const int64_t tb = (int64_t)n * kChunk + 16 * wave + 4 * grp;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t t = tb + e;
                if (t < a.T) {
                    Tio* orow = o + ((bb * a.T + t) * a.H + hh) * dv + j0 + l16;
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) orow[16 * ct] = IO::from_f(accQ[ct][e]);
                }
            }
        }
        __syncthreads();
    };
    // unrolled by two so that the operand sets swap roles without copies
    // (a register copy of a prefetched value would wait for its load)
    Ops opa, opb;
    if (a.nt > 0) load_ops(0, opa);
    for (int n = 0; n < a.nt; n += 2) {
        step(n, opa, opb);
        if (n + 1 < a.nt) step(n + 1, opb, opa);
    }

    if (a.S_out != nullptr) {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int rt = wave * SPW + i;
            if (rt < SRT) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        a.S_out[(chain * DK + 16 * rt + 4 * grp + e) * dv + j0 + 16 * ct + l16] = accS[i][ct][e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int chunk_state_slice(int64_t nchains, int dv)
{
    // enough workgroups to cover 256 CUs while keeping the per-slice operand
    // reuse (every slice re-reads the chunk's W/Qh/P/Ktil blocks) bounded
    if (dv % 64 == 0 && nchains * (dv / 64) >= 1024) return 64;
    if (dv % 32 == 0) return 32;
    return 16;
}

template <typename Tio, int DK>
static hipError_t prep_dk(const PrepArgs& a, hipStream_t s)
{
    const int64_t nblk = a.B * a.H * (int64_t)a.nt;
    if (a.dv <= 64)
        hipLaunchKernelGGL((k_chunk_prep<Tio, DK, 4>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
    else if (a.dv <= 128)
        hipLaunchKernelGGL((k_chunk_prep<Tio, DK, 8>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((k_chunk_prep<Tio, DK, 16>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename Tio>
static hipError_t prep_t(const PrepArgs& a, int dk, hipStream_t s)
{
    switch (dk) {
        case 16: return prep_dk<Tio, 16>(a, s);
        case 32: return prep_dk<Tio, 32>(a, s);
        case 64: return prep_dk<Tio, 64>(a, s);
        case 128: return prep_dk<Tio, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_prep(const PrepArgs& a, int dk, bool bf16, hipStream_t s)
{
    return bf16 ? prep_t<__bf16>(a, dk, s) : prep_t<float>(a, dk, s);
}

template <typename Tio, int DK, int VS>
static hipError_t state_v(const StateArgs& a, hipStream_t s)
{
    const int64_t nblk = a.B * a.H * (int64_t)a.nslices;
    hipLaunchKernelGGL((k_chunk_state<Tio, DK, VS>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename Tio, int DK>
static hipError_t state_dk(const StateArgs& a, int vs, hipStream_t s)
{
    switch (vs) {
        case 16: return state_v<Tio, DK, 16>(a, s);
        case 32: return state_v<Tio, DK, 32>(a, s);
        case 64: return state_v<Tio, DK, 64>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename Tio>
static hipError_t state_t(const StateArgs& a, int dk, int vs, hipStream_t s)
{
    switch (dk) {
        case 16: return state_dk<Tio, 16>(a, vs, s);
        case 32: return state_dk<Tio, 32>(a, vs, s);
        case 64: return state_dk<Tio, 64>(a, vs, s);
        case 128: return state_dk<Tio, 128>(a, vs, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_state(const StateArgs& a, int dk, int vs, bool bf16, hipStream_t s)
{
    return bf16 ? state_t<__bf16>(a, dk, vs, s) : state_t<float>(a, dk, vs, s);
}

}  // namespace gdn2
