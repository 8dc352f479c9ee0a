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

template <typename Tio, int DK>
__global__ __launch_bounds__(kThreads, 2) void k_chunk_prep(PrepArgs a)
{
    using IO = Io<Tio>;
    using SM = PrepSmem<Tio, DK>;
    constexpr int EPL = SM::EPL, KB = SM::KB, KPAD = SM::KPAD, RS = SM::RS, TS = SM::TS, FS = SM::FS;
    constexpr int ITEMS = (DK * 4 + kThreads - 1) / kThreads;
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

    // ---- 1a. running decay products inside each 16-token block -------------
    float gpre[ITEMS][16];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int item = tid + it * kThreads;
        if (item < DK * 4) {
            const int c = item % DK, p = item / DK;
            float run = 1.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 16 * p + i;
                const float al = (r < L) ? a.alpha[(row0 + r * H) * DK + c] : 1.f;
                run *= al;
                gpre[it][i] = run;
            }
            Zs[p * DK + c] = run;
        }
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
    for (int c = tid; c < DK; c += kThreads) {
        const float z0 = Zs[c], z1 = Zs[DK + c], z2 = Zs[2 * DK + c], z3 = Zs[3 * DK + c];
        Fs[0 * KPAD + c] = z0;            // pair (1,0)
        Fs[1 * KPAD + c] = z1;            // pair (2,1)
        Fs[2 * KPAD + c] = z2;            // pair (3,2)
        Fs[3 * KPAD + c] = z0 * z1;       // pair (2,0)
        Fs[4 * KPAD + c] = z1 * z2;       // pair (3,1)
        Fs[5 * KPAD + c] = z0 * z1 * z2;  // pair (3,0)
        gaml_out[c] = z0 * z1 * z2 * z3;
    }
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int item = tid + it * kThreads;
        if (item < DK * 4) {
            const int c = item % DK, p = item / DK;
            float pre = 1.f, post = 1.f;
#pragma unroll
            for (int K = 0; K < 4; ++K) {
                const float z = Zs[K * DK + c];
                if (K < p) pre *= z;
                if (K > p) post *= z;
            }
            const float zend = gpre[it][15];
            Tio kt[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 16 * p + i;
                const bool valid = r < L;
                const int64_t off = (row0 + r * H) * DK + c;
                const float kv = valid ? IO::to_f(k[off]) : 0.f;
                const float qv = valid ? IO::to_f(q[off]) : 0.f;
                const float bv = valid ? a.b[off] : 0.f;
                const float g = gpre[it][i];
                const float ig = fast_rcp(g);
                const float e = bv * kv;
                Xe[r * RS + c] = IO::from_f(e * g);
                Xq[r * RS + c] = IO::from_f(qv * g);
                Yd[r * RS + c] = IO::from_f(kv * ig);
                EhT[c * TS + r] = IO::from_f(e * g * pre);
                qh_out[r * KPAD + c] = IO::from_f(qv * g * pre);
                kt[i] = IO::from_f(kv * (zend * ig) * post);
            }
            typedef typename IO::frag frag;
#pragma unroll
            for (int i = 0; i < 16; i += EPL) {
                frag f;
#pragma unroll
                for (int e2 = 0; e2 < EPL; ++e2) f[e2] = kt[i + e2];
                *reinterpret_cast<frag*>(ktt_out + c * 64 + 16 * p + i) = f;
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
        for (int e = tid; e < 64 * nj; e += kThreads) {
            const int s = e / nj, jj = e - s * nj;
            float u = 0.f;
            if (s < L) {
                const int64_t off = (row0 + s * H) * a.dv + j0 + jj;
                u = a.w[off] * IO::to_f(v[off]);
            }
            UT[jj * TS + s] = IO::from_f(u);
        }
        __syncthreads();
        for (int jt = 0; jt < nj / 16; ++jt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 64 / KB; ++kb) {
                if (kb * KB <= 16 * wave + 15) {
                    const typename IO::frag fu = ld_frag(UT + (16 * jt + l16) * TS + kb * KB + grp * EPL);
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

    for (int n = 0; n < a.nt; ++n) {
        const char* blk = static_cast<const char*>(a.ws) + (chain * a.nt + n) * a.ws_block;
        const Tio* Qh = reinterpret_cast<const Tio*>(blk + LY.qh);
        const Tio* Ww = reinterpret_cast<const Tio*>(blk + LY.wwy);
        const Tio* Kt = reinterpret_cast<const Tio*>(blk + LY.ktt);
        const Tio* Pm = reinterpret_cast<const Tio*>(blk + LY.p);
        const float* Gl = reinterpret_cast<const float*>(blk + LY.gaml);
        const Tio* Ut = reinterpret_cast<const Tio*>(blk + LY.uwyt);
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
            const typename IO::frag fw = ld_frag(Ww + (16 * wave + l16) * KPAD + ko);
            const typename IO::frag fq = ld_frag(Qh + (16 * wave + l16) * KPAD + ko);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const typename IO::frag fs = ld_frag(Sb + (16 * ct + l16) * SRS + ko);
                accW[ct] = IO::mma(accW[ct], fw, fs);
                accQ[ct] = IO::mma(accQ[ct], fq, fs);
            }
        }
        // Delta = U - X_W (rows 16*wave + 4*grp + i, column 16*ct + l16)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const f32x4 u = ld_vec4(Ut + (int64_t)(j0 + 16 * ct + l16) * 64 + 16 * wave + 4 * grp);
            st_vec4(Dt + (16 * ct + l16) * DTS + 16 * wave + 4 * grp, u - accW[ct]);
        }
        __syncthreads();

        // O = X_Q + P Delta
#pragma unroll
        for (int kb = 0; kb < NKT; ++kb) {
            if (kb * KB <= 16 * wave + 15) {
                const int ko = kb * KB + grp * EPL;
                const typename IO::frag fp = ld_frag(Pm + (16 * wave + l16) * 64 + ko);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const typename IO::frag fd = ld_frag(Dt + (16 * ct + l16) * DTS + ko);
                    accQ[ct] = IO::mma(accQ[ct], fp, fd);
                }
            }
        }
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

        // S = diag(Gamma_L) S + Ktil^T Delta
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int rt = wave * SPW + i;
            if (rt < SRT) {
                const f32x4 gl = *reinterpret_cast<const f32x4*>(Gl + 16 * rt + 4 * grp);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) accS[i][ct] *= gl;
#pragma unroll
                for (int kb = 0; kb < NKT; ++kb) {
                    const int ko = kb * KB + grp * EPL;
                    const typename IO::frag fk = ld_frag(Kt + (16 * rt + l16) * 64 + ko);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        const typename IO::frag fd = ld_frag(Dt + (16 * ct + l16) * DTS + ko);
                        accS[i][ct] = IO::mma(accS[i][ct], fk, fd);
                    }
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    st_vec4(&SbT[(n + 1) & 1][(16 * ct + l16) * SRS + 16 * rt + 4 * grp], accS[i][ct]);
            }
        }
        __syncthreads();
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
    hipLaunchKernelGGL((k_chunk_prep<Tio, DK>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
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
