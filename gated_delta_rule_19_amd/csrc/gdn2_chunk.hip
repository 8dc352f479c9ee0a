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
// Decay ratios inside matrix products.  The chunk's 64 tokens form eight
// half-blocks of 8 tokens; half h takes its 4th token m_h as reference.  With
//   rho_r   = Gamma_r / Gamma_m,   sigma_s = Gamma_m / Gamma_s   (r, s in half h),
//   lambda_h, tau_h = the products of alpha over the first / last 4 tokens of h,
//   Z_h = lambda_h tau_h,
// a pair inside one half has Gamma_r/Gamma_s = rho_r sigma_s, and a pair with r
// in a later half hr than s's half hs has
//   Gamma_r/Gamma_s = (rho_r lambda_hr) * prod_{hs<h<hr} Z_h * (sigma_s tau_hs).
// rho and sigma are running products of at most 4 alphas or their inverses,
// so every operand of these products is bounded by the inverse product of 4
// consecutive alphas, and every correction factor is at most 1 (no exp/log is
// evaluated).  One row operand (e rho, q rho) and one column operand (k sigma)
// are stored; the per-(half, channel) corrections are applied to a fragment
// when it is loaded.  A 16x16 tile spans two halves on each side: an
// off-diagonal tile takes one product with both operands corrected, a
// diagonal tile two (same-half pairs plain, second-half rows against
// first-half columns corrected).
#include <type_traits>

#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"
#include "gdn2_layout.hpp"

namespace gdn2 {

__host__ __device__ constexpr int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr int align16(int x) { return (x + 15) & ~15; }

// ---------------------------------------------------------------------------
// k_chunk_prep
// ---------------------------------------------------------------------------
// Granule permutation of LDS rows: in a row of g 16-byte granules, granule x
// is stored at x ^ swz(row, g), so that the 16 rows one fragment read touches
// (same granule, consecutive rows) fall into distinct banks.
__host__ __device__ constexpr int swz(int row, int g)
{
    return (row / (g >= 8 ? 1 : 8 / g)) % (g >= 16 ? 16 : g);
}
// variant for rows of >= 8 granules that are also written by lanes striding 4
// rows apart (rows 4c + e): row + row/4 keeps both patterns spread
__host__ __device__ constexpr int swzu(int row, int g)
{
    return (row + row / 4) % (g >= 16 ? 16 : g);
}

template <typename Tio, int DK>
struct PrepSmem {
    static constexpr int EPL = Io<Tio>::EPL, KB = Io<Tio>::KB, ES = (int)sizeof(Tio);
    static constexpr int KPAD = round_up(DK, KB);
    static constexpr int GX = KPAD * ES / 16;   // granules per row of Xe / Xq / Yd
    static constexpr int GE = 64 * ES / 16;     // granules per row of EhT
    static constexpr int TS = 64 + EPL;         // row stride of Tm / UT (elements)
    static constexpr int SZ_X = 64 * KPAD * ES;
    static constexpr int SZ_F = 64 * 64 * 4;    // fp32 64x64, swizzled rows
    static constexpr int SZ_E = DK * 64 * ES;
    static constexpr int SZ_T = 64 * TS * ES;
    static constexpr int SZ_TD = 4 * 16 * 20 * 4;   // TD: diagonal blocks of T, row-major
    // R0: Xe -> A32 -> EhT;  R1: Xq -> T32T -> UT;  R2: Yd -> (Tm, TD)
    static constexpr int R0 = align16(imax(imax(SZ_X, SZ_F), SZ_E));
    static constexpr int SZ_U = 64 * 64 * ES;     // UT [64 columns][64 tokens], swizzled rows
    static constexpr int R1 = align16(imax(imax(SZ_X, SZ_F), SZ_U));
    static constexpr int R2 = align16(imax(SZ_X, SZ_T + SZ_TD));
    static constexpr int O1 = R0, O2 = O1 + R1, OF = O2 + R2;
    // fp32 [.][KPAD] tables of the decay corrections: lambda [8], tau [8] per
    // half; the row correction of off-diagonal tiles per half [8]; the column
    // correction per off-diagonal tile (1,0) (2,1) (3,2) (2,0) (3,1) (3,0) and
    // half of its column block [12]
    static constexpr int TL = 0, TT = 8, TRS = 16, TCS = 24, NTAB = 36;
    static constexpr int BYTES = OF + NTAB * KPAD * 4;
    // workgroups per CU the LDS and register budgets are sized for (at most 2
    // below dk 64, whose register use does not fit the budget of 3)
    static constexpr int MINB = (BYTES * 3 <= 160 * 1024 && DK >= 64) ? 3 : (BYTES * 2 <= 160 * 1024 ? 2 : 1);
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
// Tg = gate dtype (alpha, b, w): float, or __bf16 with bf16 I/O
// TOUT: the backward's layout of the block (bf16, KPAD = DK): Qh^T and P^T in
// place of Qh and P, and T, Ktil, W^T and Eh appended from a.t_off on (BwdExt)
// ---- fused short convolution ---------------------------------------------
// Its loads are issued with the other input loads, unconditionally (taps:
// conv_taps4_load / conv_taps4_pick; window rows: conv_hist_src, clamped
// addresses, values dropped afterwards with keep_or_zero).
// Source of the 4 inputs x[p, c..c+3] at position p of sequence seq: the
// tensor row `row` when p >= 0, the carried window conv_in (row p + K - 1)
// for -(K-1) <= p < 0 when it is given; else `safe` (any readable row of the
// tensor), whose value conv_hist_keep then drops (zeros: no window, or
// positions whose taps are zero).
template <typename Tio>
__device__ inline const Tio* conv_hist_src(const PrepArgs& a, const Tio* row, const Tio* safe, int64_t p, int64_t seq,
                                           int64_t c)
{
    const int K = a.conv_K;
    const bool win = p < 0 && p >= -(K - 1) && a.conv_in != nullptr;
    return p >= 0 ? row
         : win    ? static_cast<const Tio*>(a.conv_in) + (seq * (K - 1) + K - 1 + p) * a.conv_C + c
                  : safe;
}
__device__ inline bool conv_hist_keep(const PrepArgs& a, int64_t p)
{
    return p >= 0 || (p >= -(a.conv_K - 1) && a.conv_in != nullptr);
}
// x[0..7] <- conv(x) over the window (h[0..2], x[0..7]) with the taps w, in
// fp32, (optionally) through SiLU, rounded to the I/O type as a stored
// convolution output would be; tokens last to first so that x is read raw
template <typename Tio>
__device__ inline void conv8(typename Io<Tio>::vec4 (&x)[8], const typename Io<Tio>::vec4 (&h)[3], const f32x4 (&w)[4], int silu)
{
    using IO = Io<Tio>;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int j = i - 3 + m;
            z += w[m] * IO::unpack4(j >= 0 ? x[j] : h[j + 3]);
        }
        if (silu) z = z * sigmoid4(z);
        x[i] = IO::pack4(z);
    }
}

// CONV: the short convolution fused into the prologue (PrepArgs conv_*)
// (workgroups per CU: as LDS allows, at most 2 for wide values or the convolution)
template <typename Tio, int DK, int NUI, typename Tg, bool TOUT = false, bool CONV = false>
__global__ __launch_bounds__(kThreads, (((NUI <= 8 && !CONV) || (PrepSmem<Tio, DK>::MINB < 2)) ? PrepSmem<Tio, DK>::MINB : 2))
void k_chunk_prep(PrepArgs a)
{
    using IO = Io<Tio>;
    using SM = PrepSmem<Tio, DK>;
    constexpr int EPL = SM::EPL, KB = SM::KB, KPAD = SM::KPAD, TS = SM::TS, ES = SM::ES;
    constexpr int GX = SM::GX, GE = SM::GE, EPG = 16 / ES;   // EPG: elements per granule
    constexpr WsLayout LY = ws_layout(DK, 0, sizeof(Tio), KB);
    static_assert(!TOUT || (KPAD == DK && sizeof(Tio) == 2), "backward layout: bf16, no K padding");

    __shared__ __attribute__((aligned(16))) char smem[SM::BYTES];
    Tio* Xe = reinterpret_cast<Tio*>(smem);
    float* A32 = reinterpret_cast<float*>(smem);
    Tio* EhT = reinterpret_cast<Tio*>(smem);
    Tio* Xq = reinterpret_cast<Tio*>(smem + SM::O1);
    float* T32T = reinterpret_cast<float*>(smem + SM::O1);
    Tio* UT = reinterpret_cast<Tio*>(smem + SM::O1);
    Tio* Yd = reinterpret_cast<Tio*>(smem + SM::O2);
    Tio* Tm = reinterpret_cast<Tio*>(smem + SM::O2);
    float* TD = reinterpret_cast<float*>(smem + SM::O2 + SM::SZ_T);
    float* Fs = reinterpret_cast<float*>(smem + SM::OF);
    // element offsets in the swizzled arrays
    auto xo = [](int r, int c) { return r * KPAD + (((c / EPG) ^ swz(r, GX)) * EPG) + c % EPG; };   // [64][KPAD]
    auto fo = [](int r, int c) { return r * 64 + (((c / 4) ^ swz(r, 16)) * 4) + c % 4; };          // fp32 [64][64]
    // [DK][64] and [64][64] arrays written by rows 4c+e and read by rows 16t+l
    auto eo = [](int r, int c) { return r * 64 + (((c / EPG) ^ swzu(r, GE)) * EPG) + c % EPG; };     // EhT
    auto uo = [](int r, int c) { return r * 64 + (((c / EPG) ^ swzu(r, GE)) * EPG) + c % EPG; };     // UT

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    // this workgroup's chunk: value head hh, packed token index tok0 of its
    // first token, length L, workspace block chi
    const int64_t chi = blockIdx.x;
    int64_t hh, tok0;
    int64_t seq = 0, t0 = 0;                             // sequence and first position (equal lengths)
    int L;
    if (a.plan == nullptr) {
        const int64_t chain = chi / a.nt;
        const int n = (int)(chi - chain * a.nt);
        seq = chain / a.H;
        hh = chain - seq * a.H;
        t0 = (int64_t)n * kChunk;
        L = (int)((a.T - t0) < kChunk ? (a.T - t0) : kChunk);
        tok0 = seq * a.T + t0;
    } else {
        hh = chi / a.ncmax;
        const int64_t gc = chi - hh * a.ncmax;
        if (gc >= a.plan[2 * a.B + 1]) return;         // past the batch's last chunk (first[N])
        const int2 e = reinterpret_cast<const int2*>(a.plan + 2 * (a.B + 1))[gc];
        tok0 = e.x;
        L = e.y;
    }
    const int64_t H = a.H, Hk = a.Hk;
    const int64_t row0 = tok0 * H + hh;                  // row of the chunk's first token in [.,Hv,*]
    const int64_t row0k = tok0 * Hk + hh / (H / Hk);     // its q/k row in [.,H,dk]
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
    const BwdExt BX = bwd_ext(a.t_off, DK);      // (TOUT only)
    Tio* kn_out = reinterpret_cast<Tio*>(blk + BX.kn);
    Tio* wt_out = reinterpret_cast<Tio*>(blk + BX.wt);
    Tio* eh_out = reinterpret_cast<Tio*>(blk + BX.eh);

    typedef typename IO::frag frag;

    // ---- 0. key-axis loads ----------------------------------------------------
    // Inputs are read once, with nontemporal (streaming) loads: they then do
    // not displace the workspace blocks this launch writes from the last-level
    // cache, and the state pass that follows finds most of them there.
    // One vector-memory counter tracks loads and stores alike, so a load
    // issued after a store would also wait for that store to complete: every
    // load needed before the first global store is issued here.  Loads are
    // unconditional (rows past the sequence end are clamped to its last row
    // and replaced by identity tokens afterwards): a load under a branch would
    // be waited for at the join.  16-byte accesses keep the count of loads per
    // lane under the 63 the counter can track.
    // Key-axis item = (4 channels c0..c0+3, 8-token group rg).
    constexpr int NQ = DK / 4;
    const bool kact = tid < 2 * DK;
    const int cq = tid % NQ, rg = (tid / NQ) & 7, c0 = 4 * cq;
    typedef typename GateVec<Tg>::type gvec;
    const Tg* galpha = static_cast<const Tg*>(a.alpha);
    const Tg* gb = static_cast<const Tg*>(a.b);
    gvec alr[8], btr[8];
    typename IO::vec4 kk[8], qq[8];
    // (CONV) the 3 inputs before the thread's 8 tokens (before the sequence:
    // the carried window) and its channels' raw taps, requested first
    typename IO::vec4 hq[CONV ? 3 : 1], hk3[CONV ? 3 : 1];
    f32x4 tq[CONV ? 4 : 1], tk[CONV ? 4 : 1];
    if constexpr (CONV) {
        const int64_t ccq = (hh / (H / Hk)) * DK + c0, cck = Hk * DK + ccq;
        conv_taps4_load(a.conv_w, ccq, a.conv_K, tq);
        conv_taps4_load(a.conv_w, cck, a.conv_K, tk);
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            // r < 0 reads the previous chunk's rows (t0 + r >= 0) or the window;
            // before the sequence the row index is clamped to the chunk's first row
            const int r = 8 * rg - 3 + m;
            const int rr = r < L ? (t0 + r >= 0 ? r : 0) : L - 1;
            const int64_t rowq = (row0k + (int64_t)rr * Hk) * DK + c0, safe = row0k * DK + c0;
            hq[m] = *reinterpret_cast<const typename IO::vec4*>(conv_hist_src<Tio>(a, q + rowq, q + safe, t0 + r, seq, ccq));
            hk3[m] = *reinterpret_cast<const typename IO::vec4*>(conv_hist_src<Tio>(a, k + rowq, k + safe, t0 + r, seq, cck));
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 8 * rg + i;
        const int rc = r < L ? r : L - 1;
        const int64_t off = (row0 + rc * H) * DK + c0, offk = (row0k + rc * Hk) * DK + c0;
        alr[i] = __builtin_nontemporal_load(reinterpret_cast<const gvec*>(galpha + off));
        btr[i] = __builtin_nontemporal_load(reinterpret_cast<const gvec*>(gb + off));
        kk[i] = __builtin_nontemporal_load(reinterpret_cast<const typename IO::vec4*>(k + offk));
        qq[i] = __builtin_nontemporal_load(reinterpret_cast<const typename IO::vec4*>(q + offk));
    }
    if constexpr (CONV) {
        // the short convolution of q and k over the thread's 8 tokens
        f32x4 wq[4], wk[4];
        conv_taps4_pick(a.conv_K, tq, wq);
        conv_taps4_pick(a.conv_K, tk, wk);
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const bool keep = conv_hist_keep(a, t0 + 8 * rg - 3 + m);
            hq[m] = keep_or_zero(hq[m], keep);
            hk3[m] = keep_or_zero(hk3[m], keep);
        }
        conv8<Tio>(qq, hq, wq, a.conv_silu);
        conv8<Tio>(kk, hk3, wk, a.conv_silu);
    }
    // prologue: gate activations, q/k L2 norms (sum of squares over the NQ
    // lanes that hold one token's channels)
    f32x4 al[8], bt[8];
    const bool logits = (a.flags & kFlagGateLogits) != 0;
    const float bscale = (a.flags & kFlagNegEigval) ? 2.f : 1.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        al[i] = widen4(alr[i]);
        bt[i] = widen4(btr[i]);
        if (logits) {
            al[i] = sigmoid4(al[i]);
            bt[i] = sigmoid4(bt[i]) * bscale;
        }
        al[i] = alpha_floor4(al[i]);
    }
    float sk[8], sq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sk[i] = sq[i] = 1.f;
    if (a.flags & kFlagQkL2norm) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 kv = IO::unpack4(kk[i]), qv = IO::unpack4(qq[i]);
            float k2 = kv[0] * kv[0] + kv[1] * kv[1] + kv[2] * kv[2] + kv[3] * kv[3];
            float q2 = qv[0] * qv[0] + qv[1] * qv[1] + qv[2] * qv[2] + qv[3] * qv[3];
#pragma unroll
            for (int off = 1; off < NQ; off <<= 1) {
                k2 += __shfl_xor(k2, off, 64);
                q2 += __shfl_xor(q2, off, 64);
            }
            sk[i] = __builtin_amdgcn_rsqf(k2 + kL2normEps);
            sq[i] = __builtin_amdgcn_rsqf(q2 + kL2normEps);
        }
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

    // ---- 1a. decay products inside the thread's half (its 8 tokens) ----------
    // suf[i] = prod_{i<j<=7} alpha_j, inc[i] = prod_{j<=i} alpha_j; lambda and
    // tau are the products over tokens 0..3 and 4..7; rho, sigma relative to
    // token 3 (the half's 4th): P_i = prod_{i<j<=3} alpha_j (i <= 3),
    // Q_i = prod_{4<=j<=i} alpha_j (i >= 4).
    f32x4 suf[8], rho[8], sig[8];
    f32x4 lam, tau;
    {
        suf[7] = f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int i = 6; i >= 0; --i) suf[i] = suf[i + 1] * al[i + 1];
        f32x4 pp = {1.f, 1.f, 1.f, 1.f};                // P_i, i = 3 down to 0
#pragma unroll
        for (int i = 3; i >= 0; --i) {
            if (i < 3) pp *= al[i + 1];
            sig[i] = pp;
            rho[i] = f32x4{fast_rcp(pp[0]), fast_rcp(pp[1]), fast_rcp(pp[2]), fast_rcp(pp[3])};
        }
        lam = pp * al[0];
        f32x4 qp = {1.f, 1.f, 1.f, 1.f};                // Q_i, i = 4 up to 7
#pragma unroll
        for (int i = 4; i < 8; ++i) {
            qp *= al[i];
            rho[i] = qp;
            sig[i] = f32x4{fast_rcp(qp[0]), fast_rcp(qp[1]), fast_rcp(qp[2]), fast_rcp(qp[3])};
        }
        tau = qp;
        if (kact) {
            *reinterpret_cast<f32x4*>(Fs + (SM::TL + rg) * KPAD + c0) = lam;
            *reinterpret_cast<f32x4*>(Fs + (SM::TT + rg) * KPAD + c0) = tau;
        }
    }
    if constexpr (KPAD > DK) {   // zero the K padding of the operand arrays and tables
        for (int e = tid; e < 64 * (KPAD - DK); e += kThreads) {
            const int r = e / (KPAD - DK), c = DK + e % (KPAD - DK);
            Xe[xo(r, c)] = IO::from_f(0.f);
            Xq[xo(r, c)] = IO::from_f(0.f);
            Yd[xo(r, c)] = IO::from_f(0.f);
            qh_out[r * KPAD + c] = IO::from_f(0.f);
            wwy_out[r * KPAD + c] = IO::from_f(0.f);
        }
        for (int e = tid; e < SM::NTAB * (KPAD - DK); e += kThreads)
            Fs[(e / (KPAD - DK)) * KPAD + DK + e % (KPAD - DK)] = 0.f;
    }
    __syncthreads();

    // ---- 1b. products over the other halves, corrections, operands ----------
    // The (Gamma e)^T fragments are kept in registers and written to LDS after
    // the solve, when the space of A is free.
    constexpr int NEF = 8 / EPL;
    frag ehf[4][NEF];
    if (kact) {
        f32x4 pre = {1.f, 1.f, 1.f, 1.f}, post = pre, gaml = pre, zprev = pre, znext = pre;
        f32x4 zb[4];                                      // whole 16-token blocks
#pragma unroll
        for (int K = 0; K < 4; ++K) zb[K] = pre;
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const f32x4 z = *reinterpret_cast<const f32x4*>(Fs + (SM::TL + h) * KPAD + c0) *
                            *reinterpret_cast<const f32x4*>(Fs + (SM::TT + h) * KPAD + c0);
            if (h < rg) pre *= z;
            if (h > rg) post *= z;
            if (h == rg - 1) zprev = z;
            if (h == rg + 1) znext = z;
            zb[h >> 1] *= z;
            gaml *= z;
        }
        // row correction of off-diagonal tiles for rows in this half; column
        // corrections of the tiles (I, J), J = rg / 2 < I, for columns in this half
        *reinterpret_cast<f32x4*>(Fs + (SM::TRS + rg) * KPAD + c0) = (rg & 1) ? lam * zprev : lam;
        {
            const int J = rg >> 1;
            f32x4 F = (rg & 1) ? tau : tau * znext;
#pragma unroll
            for (int I = 1; I < 4; ++I) {
                if (I > J) {
                    const int pair = I - J == 1 ? J : (I - J == 2 ? 3 + J : 5);
                    *reinterpret_cast<f32x4*>(Fs + (SM::TCS + 2 * pair + (rg & 1)) * KPAD + c0) = F;
                    F *= zb[I];                           // the tile (I+1, J) also spans block I
                }
            }
        }
        if (rg == 0) *reinterpret_cast<f32x4*>(gaml_out + c0) = gaml;
        Tio kt[4][8], qt[4][8];
        f32x4 inc = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * rg + i;
            inc *= al[i];
            const f32x4 kv = IO::unpack4(kk[i]) * sk[i], qv = IO::unpack4(qq[i]) * sq[i];
            const f32x4 ev = bt[i] * kv;
            st_vec4(Xe + xo(r, c0), ev * rho[i]);
            st_vec4(Xq + xo(r, c0), qv * rho[i]);
            st_vec4(Yd + xo(r, c0), kv * sig[i]);
            const f32x4 gam = pre * inc;                  // Gamma_r
            const f32x4 qhv = qv * gam;
            if constexpr (!TOUT) st_vec4(qh_out + r * KPAD + c0, qhv);
            const f32x4 ehv = ev * gam, ktv = kv * suf[i] * post;
            if constexpr (TOUT) {
                st_vec4(kn_out + r * DK + c0, ktv);
                st_vec4(eh_out + r * DK + c0, ehv);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ehf[e][i / EPL][i % EPL] = IO::from_f(ehv[e]);
                kt[e][i] = IO::from_f(ktv[e]);
                qt[e][i] = IO::from_f(qhv[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int i = 0; i < 8; i += EPL) {
                frag f1, f2;
#pragma unroll
                for (int e2 = 0; e2 < EPL; ++e2) {
                    f1[e2] = kt[e][i + e2];
                    f2[e2] = qt[e][i + e2];
                }
                *reinterpret_cast<frag*>(ktt_out + (c0 + e) * 64 + 8 * rg + i) = f1;
                if constexpr (TOUT) *reinterpret_cast<frag*>(qh_out + (c0 + e) * 64 + 8 * rg + i) = f2;   // Qh^T
            }
        }
    }

    // ---- value-axis loads: u = w * v, needed from phase 5 on ----------------
    // value-axis item = (8-token group sg, 4 columns 4jq..4jq+3): a lane holds
    // 8 tokens of each of its columns, so that (w*v)^T goes to LDS as whole
    // 8-token fragments
    constexpr int NIT = NUI <= 8 ? 1 : 2;     // items per thread: 8 * dv/4 <= 256 * NIT
    gvec wr[NIT][8];
    typename IO::vec4 vr[NIT][8];
    typename IO::vec4 vh[CONV ? NIT : 1][3];      // (CONV) the 3 inputs before the item's tokens
    f32x4 wv[CONV ? NIT : 1][4];                  // (CONV) its columns' raw taps, then picked
    const Tg* gw = static_cast<const Tg*>(a.w);
    const int nvq = a.dv / 4;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int q = tid + it * kThreads;
        const int jq = q % nvq, sg = (q / nvq) & 7;
        if constexpr (CONV) {
            conv_taps4_load(a.conv_w, 2 * Hk * DK + hh * a.dv + 4 * jq, a.conv_K, wv[it]);
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const int r = 8 * sg - 3 + m;
                const int rr = r < L ? (t0 + r >= 0 ? r : 0) : L - 1;
                vh[it][m] = *reinterpret_cast<const typename IO::vec4*>(conv_hist_src<Tio>(
                    a, v + (row0 + (int64_t)rr * H) * a.dv + 4 * jq, v + row0 * a.dv + 4 * jq, t0 + r, seq,
                    2 * Hk * DK + hh * a.dv + 4 * jq));
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int s = 8 * sg + i;
            const int64_t off = (row0 + (s < L ? s : L - 1) * H) * a.dv + 4 * jq;
            wr[it][i] = __builtin_nontemporal_load(reinterpret_cast<const gvec*>(gw + off));
            vr[it][i] = __builtin_nontemporal_load(reinterpret_cast<const typename IO::vec4*>(v + off));
        }
    }
    __syncthreads();

    // ---- 2. A^T and P^T tiles on the matrix cores ---------------------------
    // tile (J, I): rows s of block J, columns r of block I,
    // D[s][r] = sum_c Y[s][c] (f_IJ[c]) X[r][c]
    // Lane l16 supplies row s = 16J + l16 of the column operand and row
    // r = 16I + l16 of the row operands; a diagonal tile adds a second product
    // with the corrections of second-half rows against first-half columns and
    // keeps it where the lane's element pairs those halves.
    f32x4 accA[3], accP[3];
#pragma unroll
    for (int pi = 0; pi < 3; ++pi) {
        accA[pi] = f32x4{0.f, 0.f, 0.f, 0.f};
        accP[pi] = accA[pi];
        const int pr = wave + 4 * pi;
        if (pr < 10) {
            const int I = unpack2(kPairI, pr), J = unpack2(kPairJ, pr);
            const int hl = l16 >> 3;
            const bool diag = pr < 4;
            // corrections: off-diagonal rows by half 2I + hl, columns by (tile, half 2J + hl);
            // the diagonal's second product rows by lambda of half 2I+1, columns by tau of half 2I
            const float* rsc = Fs + (diag ? SM::TL + 2 * I + 1 : SM::TRS + 2 * I + hl) * KPAD;
            const float* csc = Fs + (diag ? SM::TT + 2 * I : SM::TCS + 2 * (pr - 4) + hl) * KPAD;
            f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, p1 = a1;
#pragma unroll
            for (int kb = 0; kb < KPAD / KB; ++kb) {
                const int ko = kb * KB + grp * EPL;
                const typename IO::frag y = ld_frag(Yd + xo(16 * J + l16, ko));
                const typename IO::frag xe = ld_frag(Xe + xo(16 * I + l16, ko));
                const typename IO::frag xq = ld_frag(Xq + xo(16 * I + l16, ko));
                const typename IO::frag ys = IO::scale(y, csc + ko);
                const typename IO::frag xes = IO::scale(xe, rsc + ko);
                const typename IO::frag xqs = IO::scale(xq, rsc + ko);
                if (diag) {
                    accA[pi] = IO::mma(accA[pi], y, xe);
                    if constexpr (TOUT) accP[pi] = IO::mma(accP[pi], xq, y);   // D[r][s]
                    else accP[pi] = IO::mma(accP[pi], y, xq);
                }
                a1 = IO::mma(a1, ys, xes);
                if constexpr (TOUT) p1 = IO::mma(p1, xqs, ys);
                else p1 = IO::mma(p1, ys, xqs);
            }
            // accumulator element e: D[s = 4grp + e][r = l16] (TOUT's P: D[r = 4grp + e][s = l16])
            if (!diag) {
                accA[pi] = a1;
                accP[pi] = p1;
            } else {
                if (l16 >= 8 && grp < 2) accA[pi] = a1;            // r second half, s first half
                if (TOUT ? (l16 < 8 && grp >= 2) : (l16 >= 8 && grp < 2)) accP[pi] = p1;
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
                    if (TOUT ? l16 > s : s > l16) pv[i] = 0.f;    // TOUT: pv[i] = P[16I+4grp+i][16J+l16]
                }
            }
            *reinterpret_cast<f32x4*>(A32 + fo(r, 16 * J + 4 * grp)) = av;
            if constexpr (TOUT) st_vec4(p_out + (16 * J + l16) * 64 + 16 * I + 4 * grp, pv);   // P^T
            else st_vec4(p_out + r * 64 + 16 * J + 4 * grp, pv);
        }
    }
    for (int u = wave; u < 6; u += 4) {   // P is zero above the block diagonal (P^T below it)
        const int I = unpack2(kUpperI, u), J = unpack2(kUpperJ, u);
        if constexpr (TOUT) st_vec4(p_out + (16 * J + l16) * 64 + 16 * I + 4 * grp, f32x4{0.f, 0.f, 0.f, 0.f});
        else st_vec4(p_out + (16 * I + l16) * 64 + 16 * J + 4 * grp, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    __syncthreads();

    // ---- 3. T = (I + A)^{-1}, fp32 -------------------------------------------
    // Diagonal 16x16 blocks by forward substitution (one lane per column);
    // then, block row by block row, T[I][J] = -T_II (A[I][0:I] T[0:I][J]) on
    // fp32 matrix cores: the first product's accumulator is already laid out
    // as the second product's B operand.  T is kept transposed (T32T[n][s],
    // K index contiguous) for the B operands, the diagonal blocks row-major
    // (TD) for the A operands, and in the I/O dtype (Tm) for phases 4 and 5.
    using F32 = Io<float>;
    if (wave == 0) {
        const int I = lane >> 4, j = lane & 15;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int sp = 0; sp < r; ++sp) acc -= A32[fo(16 * I + r, 16 * I + sp)] * x[sp];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            TD[(I * 16 + r) * 20 + j] = x[r];
            Tm[(16 * I + r) * TS + 16 * I + j] = IO::from_f(x[r]);
        }
#pragma unroll
        for (int r = 0; r < 16; r += 4)
            *reinterpret_cast<f32x4*>(T32T + fo(16 * I + j, 16 * I + r)) = f32x4{x[r], x[r + 1], x[r + 2], x[r + 3]};
    } else {
        // blocks of T above the diagonal are zero (T32T only ever reads the
        // blocks on or below it)
        for (int e = tid - 64; e < 6 * 256; e += kThreads - 64) {
            const int u = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
            const int bi = unpack2(kUpperI, u), bj = unpack2(kUpperJ, u);
            Tm[(16 * bi + rr) * TS + 16 * bj + cc] = IO::from_f(0.f);
        }
    }
    __syncthreads();
#pragma unroll
    for (int I = 1; I < 4; ++I) {
        if (wave < I) {
            const int J = wave;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kb = J; kb < I; ++kb) {
                const f32x4 fa = *reinterpret_cast<const f32x4*>(A32 + fo(16 * I + l16, 16 * kb + 4 * grp));
                const f32x4 fb = *reinterpret_cast<const f32x4*>(T32T + fo(16 * J + l16, 16 * kb + 4 * grp));
                acc = F32::mma(acc, fa, fb);
            }
            const f32x4 ft = *reinterpret_cast<const f32x4*>(TD + (I * 16 + l16) * 20 + 4 * grp);
            const f32x4 t4 = -F32::mma(f32x4{0.f, 0.f, 0.f, 0.f}, ft, acc);
            // t4[e] = T[16I + 4grp + e][16J + l16]
            *reinterpret_cast<f32x4*>(T32T + fo(16 * J + l16, 16 * I + 4 * grp)) = t4;
#pragma unroll
            for (int e = 0; e < 4; ++e) Tm[(16 * I + 4 * grp + e) * TS + 16 * J + l16] = IO::from_f(t4[e]);
        }
        __syncthreads();
    }
    // (Gamma e)^T into the space of A
    if (kact) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < NEF; ++i)
                *reinterpret_cast<frag*>(EhT + eo(c0 + e, 8 * rg + EPL * i)) = ehf[e][i];
    }
    __syncthreads();

    // ---- 4. W^T = (Gamma e)^T T^T : tile (c-block, r-block = wave) ----------
    typename IO::frag tf[64 / KB];
#pragma unroll
    for (int kb = 0; kb < 64 / KB; ++kb) tf[kb] = ld_frag(Tm + (16 * wave + l16) * TS + kb * KB + grp * EPL);
    if constexpr (TOUT) {
        Tio* t_out = reinterpret_cast<Tio*>(blk + a.t_off);
#pragma unroll
        for (int kb = 0; kb < 64 / KB; ++kb)
            *reinterpret_cast<frag*>(t_out + (16 * wave + l16) * 64 + kb * KB + grp * EPL) = tf[kb];
    }
#pragma unroll
    for (int ct = 0; ct < DK / 16; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 64 / KB; ++kb) {
            if (kb * KB <= 16 * wave + 15) {
                const typename IO::frag fe = ld_frag(EhT + eo(16 * ct + l16, kb * KB + grp * EPL));
                acc = IO::mma(acc, fe, tf[kb]);
            }
        }
        // acc[i] = W[r = 16*wave + l16][c = 16*ct + 4*grp + i]
        st_vec4(wwy_out + (16 * wave + l16) * KPAD + 16 * ct + 4 * grp, acc);
        if constexpr (TOUT) {
            // W^T: after a transpose inside each lane quad, lane q holds
            // W[16*wave + (l16 & ~3) + e][16*ct + 4*grp + q], e = 0..3
            const f32x4 t = quad_transpose4(acc);
            st_vec4(wt_out + (16 * ct + 4 * grp + (l16 & 3)) * 64 + 16 * wave + (l16 & ~3), t);
        }
    }

    // ---- 5. U = T (w * v), stored transposed, in column blocks of 64 --------
    // (w*v) of tokens past the sequence end is zero
    frag uf[NIT][4][8 / EPL];      // per item and column: the 8 tokens as fragments
    if constexpr (CONV) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int sg = ((tid + it * kThreads) / nvq) & 7;
            f32x4 wp[4];
            conv_taps4_pick(a.conv_K, wv[it], wp);
#pragma unroll
            for (int m = 0; m < 3; ++m) vh[it][m] = keep_or_zero(vh[it][m], conv_hist_keep(a, t0 + 8 * sg - 3 + m));
            conv8<Tio>(vr[it], vh[it], wp, a.conv_silu);
        }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int sg = ((tid + it * kThreads) / nvq) & 7;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 w4 = logits ? sigmoid4(widen4(wr[it][i])) : widen4(wr[it][i]);
            const f32x4 u4 = (8 * sg + i < L) ? w4 * IO::unpack4(vr[it][i]) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) uf[it][e][i / EPL][i % EPL] = IO::from_f(u4[e]);
        }
    }
    for (int j0 = 0; j0 < a.dv; j0 += 64) {
        const int nj = (a.dv - j0) < 64 ? (a.dv - j0) : 64;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int q = tid + it * kThreads;
            const int c = 4 * (q % nvq) - j0, sg = q / nvq;
            if (sg < 8 && c >= 0 && c < nj) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int f = 0; f < 8 / EPL; ++f)
                        *reinterpret_cast<frag*>(UT + uo(c + e, 8 * sg + EPL * f)) = uf[it][e][f];
            }
        }
        __syncthreads();
        for (int jt = 0; jt < nj / 16; ++jt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 64 / KB; ++kb) {
                if (kb * KB <= 16 * wave + 15) {
                    const frag fu = ld_frag(UT + uo(16 * jt + l16, kb * KB + grp * EPL));
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
// Workgroup = (batch, head, slice of VS value columns), 8 waves: 4 compute
// waves and 4 loader waves.
//
// Compute waves: the slice of S (DK x VS, fp32) lives in matrix-core
// accumulators; compute wave w owns state row tiles [w*SPW, (w+1)*SPW) and
// token block w of every chunk.  Per chunk:
//   X_W = W S          (rows: token block w; B operand: S^T copy in LDS)
//   Delta = U - X_W    -> LDS (transposed)                      | barrier 1
//   O^T = S^T Qh^T + Delta^T P^T   (lanes hold 4 adjacent columns of one
//                                   token, so o is written 4 columns at a time)
//   S = diag(Gamma_L) S + Ktil^T Delta  -> LDS copy of S for the next chunk
//                                                               | barrier 2
// Loader waves keep the next three chunks' factors (W, Qh, P, Ktil^T,
// Gamma_L and this slice's U^T) in flight in their own registers and copy
// chunk n+1 into the second LDS buffer while chunk n is computed, so the
// memory latency of a chunk is hidden behind three chunks of compute.  In
// LDS every factor row is stored with its 16-byte granules XOR-permuted by
// the row index so that the 16 rows a fragment read touches fall into
// distinct banks.  LDS operands of a stage are read before its products.
// The slices of one head get block ids congruent mod 8 so that they run on
// one XCD and fetch the head's workspace blocks through a single L2.

// value columns per compute wave, loader waves per workgroup
#ifndef GDN2_STATE_CW
#define GDN2_STATE_CW 32
#endif
// loader waves: 8, or 4 where the workgroup already has 8 compute waves or
// fp32 operands (their registers would not fit beside eight loaders)
__host__ __device__ constexpr int state_cw(int vs) { return vs < GDN2_STATE_CW ? vs : GDN2_STATE_CW; }
__host__ __device__ constexpr int state_nlw(int vs, int es) { return (vs / state_cw(vs) > 1 || es == 4) ? 4 : 8; }
__host__ __device__ constexpr int state_threads(int vs, int es) { return 64 * (4 * (vs / state_cw(vs)) + state_nlw(vs, es)); }

// NOQ: the checkpointing pass, which writes no o and needs neither Qh nor P
template <typename Tio, int DK, int VS, bool NOQ = false>
struct StateLds {
    static constexpr int ES = (int)sizeof(Tio), KB = Io<Tio>::KB, EPL = Io<Tio>::EPL;
    static constexpr int KPAD = round_up(DK, KB);
    static constexpr int GW = KPAD * ES / 16;       // granules per row of W / Qh
    static constexpr int GT = 64 * ES / 16;         // granules per row of P / Ktil^T / U^T
    // granule offsets of the sections of one operand buffer (Qh and P empty with NOQ)
    static constexpr int NQ = NOQ ? 0 : 1;
    static constexpr int O_W = 0, O_Q = O_W + 64 * GW, O_P = O_Q + NQ * 64 * GW, O_K = O_P + NQ * 64 * GT;
    static constexpr int O_U = O_K + DK * GT, O_G = O_U + VS * GT, GBUF = O_G + DK / 4;
    static constexpr int SRS = KPAD + EPL, DTS = 64 + EPL;
    // NOQ (bf16, dk a multiple of 32): the state also row-major, [DK][SP],
    // for the checkpoint copy
    static constexpr bool CKL = NOQ && ES == 2 && DK % 32 == 0;
    static constexpr int SP = VS + 16 / ES;
    static constexpr int PRIV = VS * SRS * ES + VS * DTS * ES + (CKL ? DK * SP * ES : 0);
    static constexpr int LIMIT = 160 * 1024;
    // two operand buffers when they fit (loads of chunk n+1 overlap chunk n),
    // else one (the copy waits for the chunk to finish: one more barrier)
    static constexpr int NB = (2 * GBUF * 16 + PRIV <= LIMIT) ? 2 : 1;
    static constexpr bool FITS = GBUF * 16 + PRIV <= LIMIT;
    static constexpr int BYTES = NB * GBUF * 16 + PRIV;
    static constexpr int NLD = 64 * state_nlw(VS, ES);   // loader lanes
    static constexpr int LPL = (GBUF + NLD - 1) / NLD;   // granules per loader lane per chunk
};

// bytes of LDS the state kernel needs for (dk, slice width, element size),
// or 0 when it does not fit (mirrors StateLds for the host)
inline int state_lds_bytes(int dk, int vs, int es)
{
    const int kb = es == 2 ? 32 : 16;
    const int kpad = (dk + kb - 1) / kb * kb;
    const int gw = kpad * es / 16, gt = 64 * es / 16;
    const int gbuf = 64 * gw * 2 + 64 * gt + dk * gt + vs * gt + dk / 4;
    const int priv = vs * (kpad + 16 / es) * es + vs * (64 + 16 / es) * es;
    if (2 * gbuf * 16 + priv <= 160 * 1024) return 2 * gbuf * 16 + priv;
    if (gbuf * 16 + priv <= 160 * 1024) return gbuf * 16 + priv;
    return 0;
}

// The fused short convolution's window after the last token (StateArgs
// conv_*, equal-length batches): the first slice of each chain copies the
// last conv_K-1 inputs of its value head's columns, and of its query/key
// head when it is the group's first value head, into conv_out.  The state
// pass runs after the prep has read every input it needs, and here all reads
// come before all writes (a barrier between), so conv_out may be conv_in.
// Called by every thread of the workgroup.
template <typename Tio, int DK>
__device__ void conv_window_out(const StateArgs& a, int64_t bb, int64_t hh)
{
    using IO = Io<Tio>;
    constexpr int MAXE = 4;                       // elements per thread (3 rows of 2 dk + dv <= 768)
    const int K1 = a.conv_K - 1, nt = blockDim.x, tid = threadIdx.x;
    const int64_t G = a.H / a.Hk, hk = hh / G;
    const int nqk = (hh % G) == 0 ? 2 * DK : 0, nch = nqk + a.dv;
    Tio val[MAXE];
    int64_t dst[MAXE];
#pragma unroll
    for (int m = 0; m < MAXE; ++m) {
        const int e = tid + m * nt;
        dst[m] = -1;
        if (e < K1 * nch) {
            const int j = e / nch, ch = e - j * nch;
            const int64_t p = a.T - K1 + j;       // position of row j of the window
            int64_t c;
            const Tio* src;
            if (ch < nqk) {
                const int which = ch / DK, cc = ch - which * DK;
                c = which * a.Hk * DK + hk * DK + cc;
                src = static_cast<const Tio*>(which == 0 ? a.cq : a.ck) + ((bb * a.T + p) * a.Hk + hk) * DK + cc;
            } else {
                const int col = ch - nqk;
                c = 2 * a.Hk * DK + hh * a.dv + col;
                src = static_cast<const Tio*>(a.cv) + ((bb * a.T + p) * a.H + hh) * a.dv + col;
            }
            if (p >= 0) val[m] = *src;
            else if (a.conv_in != nullptr) val[m] = static_cast<const Tio*>(a.conv_in)[(bb * K1 + K1 + p) * a.conv_C + c];
            else val[m] = IO::from_f(0.f);
            dst[m] = (bb * K1 + j) * a.conv_C + c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MAXE; ++m)
        if (dst[m] >= 0) static_cast<Tio*>(a.conv_out)[dst[m]] = val[m];
}

// value columns per compute wave and threads per workgroup of the state pass

// CHK: write the state entering every chunk (the checkpoints of StateArgs)
// instead of o: Qh and P are neither copied nor used
template <typename Tio, int DK, int VS, bool CHK>
__global__ __launch_bounds__(state_threads(VS, (int)sizeof(Tio)), 1) void k_chunk_state(StateArgs a)
{
    using IO = Io<Tio>;
    using L = StateLds<Tio, DK, VS, CHK>;
    typedef typename IO::frag frag;
    typedef typename IO::vec4 vec4;
    constexpr int EPL = IO::EPL, KB = IO::KB, ES = L::ES;
    constexpr int KPAD = L::KPAD, GW = L::GW, GT = L::GT;
    constexpr int CW = state_cw(VS);               // columns per compute wave
    constexpr int NCH = VS / CW;                   // column groups: compute waves = 4 * NCH
    constexpr int NCW = 4 * NCH;
    constexpr int NCT = CW / 16;                   // column tiles per compute wave
    constexpr int SRT = DK / 16;
    constexpr int SPW = (SRT + 3) / 4;
    constexpr int SRS = L::SRS, DTS = L::DTS;
    constexpr int NKX = KPAD / KB;
    constexpr int NKT = 64 / KB;
    constexpr int GB = KB * ES / 16;                // granules per K-block
    constexpr int LPL = L::LPL;
    constexpr WsLayout LY = ws_layout(DK, 0, sizeof(Tio), KB);
    constexpr int NB = L::NB;
    static_assert(L::FITS && L::BYTES <= L::LIMIT, "LDS budget");

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    Tio* SbT = reinterpret_cast<Tio*>(smem + NB * L::GBUF * 16);            // S^T      [j][c]
    Tio* DT = reinterpret_cast<Tio*>(smem + NB * L::GBUF * 16 + VS * SRS * ES);  // Delta^T  [j][s]
    Tio* SN = reinterpret_cast<Tio*>(smem + NB * L::GBUF * 16 + VS * (SRS + DTS) * ES);   // S [c][j] (CHK, bf16)
    // the checkpoints in the I/O dtype are copied from LDS by the loader waves
    constexpr bool CKL = L::CKL;
    constexpr int SP = L::SP;

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool loader = wave >= NCW;
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
    const int64_t bb = chain / a.H, hh = chain - bb * a.H;   // sequence, value head
    const int dv = a.dv;
    if (a.conv_out != nullptr && a.conv_K > 1 && slice == 0) conv_window_out<Tio, DK>(a, bb, hh);
    // the sequence's first packed token, its length, chunk count and first
    // workspace block (checkpoints follow the blocks)
    const ChainSpan sp = chain_span(a.plan, a.ncmax, a.B, a.T, a.H, a.nt, bb, hh);
    const int64_t tok0 = sp.tok0, tlen = sp.tlen, blk0 = sp.blk0;
    const int nt = sp.nt;
    const char* wsbase = static_cast<const char*>(a.ws) + blk0 * a.ws_block;

    if (loader) {
        // ---------------- loader waves ------------------------------------
        // granule g = (wave - NCW)*64 + lane + NLD*m of a buffer: source offset
        // in the workspace block and destination in the buffer (constant per chunk)
        int src[LPL], dst[LPL];
#pragma unroll
        for (int m = 0; m < LPL; ++m) {
            int g = (wave - NCW) * 64 + lane + L::NLD * m;
            // idle slots copy a granule some other lane copies too (the same
            // bytes to the same place); distinct addresses keep their loads
            // and LDS writes spread over banks instead of piling onto one
            g %= L::GBUF;
            // granule x of a section whose rows hold GPR granules (compile-time
            // widths keep the index arithmetic to shifts and masks); stored
            // granule = (row, column ^ swz(row))
            auto map = [&](int x, auto gpr_c, int sec_src, int sec_base) {
                constexpr int GPR = decltype(gpr_c)::value;
                const int row = x / GPR, gr = x % GPR;
                src[m] = sec_src + row * (GPR * 16) + gr * 16;
                dst[m] = (sec_base + row * GPR + (gr ^ swz(row, GPR))) * 16;
            };
            using cGW = std::integral_constant<int, GW>;
            using cGT = std::integral_constant<int, GT>;
            if (g < L::O_Q)      map(g - L::O_W, cGW{}, (int)LY.wwy, L::O_W);
            else if (g < L::O_P) map(g - L::O_Q, cGW{}, (int)LY.qh, L::O_Q);
            else if (g < L::O_K) map(g - L::O_P, cGT{}, (int)LY.p, L::O_P);
            else if (g < L::O_U) map(g - L::O_K, cGT{}, (int)LY.ktt, L::O_K);
            else if (g < L::O_G) map(g - L::O_U, cGT{}, (int)LY.uwyt + j0 * 64 * ES, L::O_U);
            else { src[m] = (int)LY.gaml + (g - L::O_G) * 16; dst[m] = g * 16; }
        }
        // register slots of chunks in flight: as many (up to five) as fit in
        // the registers a lane has next to the compute waves' budget, less
        // what the checkpoint copy holds (measured: no spills)
        constexpr int NW = NCW + state_nlw(VS, ES);
        constexpr int WAVES_PER_SIMD = (NW + 3) / 4;
        constexpr int NCKI = (VS * DK * ES / 16 + DK * VS * ES / 16 + L::NLD - 1) / L::NLD;   // copy rounds
        constexpr int CKREG = CKL ? (NCKI <= 2 ? 64 : 96) : 0;
        constexpr int VBUDGET = (WAVES_PER_SIMD <= 2 ? 256 : (WAVES_PER_SIMD == 3 ? 168 : 128)) - 2 * LPL - 16 - CKREG;
        constexpr int DEPTH0 = VBUDGET / (4 * LPL);
        constexpr int DEPTH = DEPTH0 > 5 ? 5 : (DEPTH0 < 1 ? 1 : DEPTH0);
        frag r[DEPTH][LPL];
        // granules [m0, m1) of chunk n into / out of a register slot
        auto fetch = [&](int n, frag* rs, int m0, int m1) {
            const char* blk = wsbase + (int64_t)(n < nt ? n : nt - 1) * a.ws_block;
#pragma unroll
            for (int m = 0; m < LPL; ++m)
                if (m >= m0 && m < m1) rs[m] = *reinterpret_cast<const frag*>(blk + src[m]);
        };
        auto store = [&](int buf, const frag* rs, int m0, int m1) {
            char* b0 = smem + buf * L::GBUF * 16;
#pragma unroll
            for (int m = 0; m < LPL; ++m)
                if (m >= m0 && m < m1) *reinterpret_cast<frag*>(b0 + dst[m]) = rs[m];
        };
        // Chunk c travels in slot c % DEPTH.  Iteration n: chunk n+1 goes to
        // LDS and chunk n+1+DEPTH is requested into the slot it leaves, half
        // before barrier 1 and half after it, so that the copy overlaps both
        // compute phases and barrier 1 (which orders the compute waves' Delta
        // exchange) does not wait for the whole copy.  Every iteration issues
        // the same loads and stores (chunk numbers past the end are clamped,
        // and a copy past the end lands in the buffer no one reads any more):
        // with no conditional fetch the compiler can count exactly how many
        // loads are still in flight behind the ones a store needs, so the
        // stores wait only for their own chunk, DEPTH iterations old.
        // the state entering chunk n, from LDS (S^T and S, bf16) to the
        // checkpoints [dv][dk] and [dk][dv]; runs before barrier 1 of chunk n,
        // while the compute waves only read both copies
        auto ckpt = [&](int n) {
            if constexpr (CKL) {
                constexpr int GR = DK * ES / 16, GN = VS * ES / 16, EG = 16 / ES;
                constexpr int G1 = VS * GR, G2 = DK * GN;
                const int64_t cb = (blk0 + n) * DK * dv;
#pragma unroll
                for (int q0 = 0; q0 < G1 + G2; q0 += L::NLD) {
                    const int q = q0 + (wave - NCW) * 64 + lane;
                    if (q < G1) {
                        const int j = q / GR, c = (q % GR) * EG;
                        const f32x4 v = *reinterpret_cast<const f32x4*>(SbT + j * SRS + c);
                        if (a.S_chkT != nullptr)
                            *reinterpret_cast<f32x4*>(static_cast<Tio*>(a.S_chkT) + cb + (int64_t)(j0 + j) * DK + c) = v;
                    } else if (q < G1 + G2) {
                        const int c = (q - G1) / GN, jj = ((q - G1) % GN) * EG;
                        const f32x4 v = *reinterpret_cast<const f32x4*>(SN + c * SP + jj);
                        if (a.S_chkIo != nullptr)
                            *reinterpret_cast<f32x4*>(static_cast<Tio*>(a.S_chkIo) + cb + (int64_t)c * dv + j0 + jj) = v;
                    }
                }
            }
        };
        constexpr int HALF = LPL / 2;
        auto iter = [&](int n, frag* rs) {
            ckpt(n);
            if (NB == 2) {
                store((n + 1) & 1, rs, 0, HALF);
                fetch(n + 1 + DEPTH, rs, 0, HALF);
                __syncthreads();                          // barrier 1
                store((n + 1) & 1, rs, HALF, LPL);
                fetch(n + 1 + DEPTH, rs, HALF, LPL);
                __syncthreads();                          // barrier 2
            } else {
                __syncthreads();                          // barrier 1
                __syncthreads();                          // barrier 2: chunk n done
                store(0, rs, 0, LPL);
                fetch(n + 1 + DEPTH, rs, 0, LPL);
                __syncthreads();                          // barrier 3: buffer refilled
            }
        };
        if (nt == 0) {                                    // state copy only
            __syncthreads();                              // prologue barrier
            return;
        }
        // chunk 0 first: the compute waves start as soon as it is in LDS
        fetch(0, r[0], 0, LPL);
        if (DEPTH > 1) fetch(1, r[DEPTH > 1 ? 1 : 0], 0, LPL);
        store(0, r[0], 0, LPL);
        __syncthreads();                                  // prologue barrier
#pragma unroll
        for (int d = 2; d < DEPTH; ++d) fetch(d, r[d], 0, LPL);
        fetch(DEPTH, r[0], 0, LPL);
        int n = 0;
        for (; n + DEPTH <= nt; n += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) iter(n + d, r[(d + 1) % DEPTH]);
        }
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d)
            if (n + d < nt) iter(n + d, r[(d + 1) % DEPTH]);
        return;
    }

    // ---------------- compute waves -------------------------------------------
    // compute wave = (token block tb, column group ch of CW columns)
    const int tb = wave & 3, ch = wave >> 2, jc = ch * CW;
    Tio* o = static_cast<Tio*>(a.o);
    f32x4 accS[SPW][NCT];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int rt = tb * SPW + i < SRT ? tb * SPW + i : SRT - 1;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (a.S0 != nullptr) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = a.S0[(chain * DK + 16 * rt + 4 * grp + e) * dv + j0 + jc + 16 * ct + l16];
            }
            accS[i][ct] = v;
        }
    }
    if constexpr (KPAD > DK) {
        for (int e = tid; e < VS * (KPAD - DK); e += 64 * NCW)
            SbT[(e / (KPAD - DK)) * SRS + DK + e % (KPAD - DK)] = IO::from_f(0.f);
    }
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int rt = tb * SPW + i;
        if (rt < SRT) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                st_vec4(&SbT[(jc + 16 * ct + l16) * SRS + 16 * rt + 4 * grp], accS[i][ct]);
                // S row-major: after a transpose inside each lane quad, lane q
                // holds row 16 rt + 4 grp + q, columns (l16 & ~3) .. +3 of the tile
                if constexpr (CKL)
                    st_vec4(&SN[(16 * rt + 4 * grp + (l16 & 3)) * SP + jc + 16 * ct + (l16 & ~3)], quad_transpose4(accS[i][ct]));
            }
        }
    }
    __syncthreads();                                      // prologue barrier

    // fragment (16 bytes) of row r, K-block kb of a swizzled section
    auto lfrag = [&](const char* sec, int r, int gpr, int kb) -> frag {
        const int g = (kb * GB + grp) ^ swz(r, gpr);
        return *reinterpret_cast<const frag*>(sec + (r * gpr + g) * 16);
    };

    for (int n = 0; n < nt; ++n) {
        if constexpr (CHK) {
            // checkpoint: the state entering chunk n (kept for the backward pass).
            // fp32 here; in bf16 the loader waves copy it from LDS.  Lanes
            // 4m .. 4m+3 of a 16-lane row hold 4 columns of 4 state rows; a
            // transpose inside each lane quad gives every lane 4 consecutive
            // columns of one row, written as one vector.
            if (a.S_chk != nullptr) {
                const int64_t base = (blk0 + n) * DK * dv + j0 + jc + (l16 & ~3);
#pragma unroll
                for (int i = 0; i < SPW; ++i) {
                    const int rt = tb * SPW + i;
                    if (rt < SRT) {
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) {
                            const f32x4 t = quad_transpose4(accS[i][ct]);
                            const int64_t o = base + (int64_t)(16 * rt + 4 * grp + (l16 & 3)) * dv + 16 * ct;
                            *reinterpret_cast<f32x4*>(a.S_chk + o) = t;
                        }
                    }
                }
            }
        }
        const char* B0 = smem + (NB == 2 ? (n & 1) : 0) * L::GBUF * 16;
        const char* Wl = B0 + L::O_W * 16;
        const char* Ql = B0 + L::O_Q * 16;
        const char* Pl = B0 + L::O_P * 16;
        const char* Kl = B0 + L::O_K * 16;
        const char* Ul = B0 + L::O_U * 16;
        const float* Gl = reinterpret_cast<const float*>(B0 + L::O_G * 16);

        // X_W = W S and O^T = S^T Qh^T
        frag fw[NKX], fq[NKX];
#pragma unroll
        for (int kb = 0; kb < NKX; ++kb) {
            fw[kb] = lfrag(Wl, 16 * tb + l16, GW, kb);
            if constexpr (!CHK) fq[kb] = lfrag(Ql, 16 * tb + l16, GW, kb);
        }
        f32x4 accW[NCT], accO[NCT];
        frag fsb[2][NKX];
#pragma unroll
        for (int kb = 0; kb < NKX; ++kb) fsb[0][kb] = ld_frag(&SbT[(jc + l16) * SRS + kb * KB + grp * EPL]);
        // operands that do not depend on this chunk's products are read now,
        // so that only the Delta reads remain behind barrier 1
        vec4 u4[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int row = jc + 16 * ct + l16, r = 16 * tb + 4 * grp;
            const int g = (r * ES / 16) ^ swz(row, GT);
            u4[ct] = *reinterpret_cast<const vec4*>(Ul + (row * GT + g) * 16 + (r * ES) % 16);
        }
        frag fp[NKT], fk[SPW][NKT];
        f32x4 gl[SPW];
#pragma unroll
        for (int kb = 0; kb < NKT; ++kb) {
            if constexpr (!CHK) fp[kb] = lfrag(Pl, 16 * tb + l16, GT, kb);
#pragma unroll
            for (int i = 0; i < SPW; ++i) {
                const int rt = tb * SPW + i < SRT ? tb * SPW + i : SRT - 1;
                fk[i][kb] = lfrag(Kl, 16 * rt + l16, GT, kb);
            }
        }
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int rt = tb * SPW + i < SRT ? tb * SPW + i : SRT - 1;
            gl[i] = *reinterpret_cast<const f32x4*>(Gl + 16 * rt + 4 * grp);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            if (ct + 1 < NCT) {
#pragma unroll
                for (int kb = 0; kb < NKX; ++kb)
                    fsb[(ct + 1) & 1][kb] = ld_frag(&SbT[(jc + 16 * (ct + 1) + l16) * SRS + kb * KB + grp * EPL]);
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x4 w4 = {0.f, 0.f, 0.f, 0.f}, o4 = w4;
#pragma unroll
            for (int kb = 0; kb < NKX; ++kb) {
                w4 = IO::mma(w4, fw[kb], fsb[ct & 1][kb]);     // D[token][col]
                if constexpr (!CHK) o4 = IO::mma(o4, fsb[ct & 1][kb], fq[kb]);     // D[col][token]
            }
            accW[ct] = w4;
            accO[ct] = o4;
        }
        // Delta = U - X_W  (rows 16*wave + 4*grp + e, column 16*ct + l16) -> DT[col][token]
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int row = jc + 16 * ct + l16, r = 16 * tb + 4 * grp;
            st_vec4(&DT[row * DTS + r], IO::unpack4(u4[ct]) - accW[ct]);
        }
        __syncthreads();                                  // barrier 1

        // O^T += Delta^T P^T;  S = diag(Gamma_L) S + Ktil^T Delta
#pragma unroll
        for (int i = 0; i < SPW; ++i)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) accS[i][ct] *= gl[i];
        frag fdb[2][NKT];
#pragma unroll
        for (int kb = 0; kb < NKT; ++kb) fdb[0][kb] = ld_frag(&DT[(jc + l16) * DTS + kb * KB + grp * EPL]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            if (ct + 1 < NCT) {
#pragma unroll
                for (int kb = 0; kb < NKT; ++kb)
                    fdb[(ct + 1) & 1][kb] = ld_frag(&DT[(jc + 16 * (ct + 1) + l16) * DTS + kb * KB + grp * EPL]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < NKT; ++kb) {
                if (!CHK && kb * KB <= 16 * tb + 15) accO[ct] = IO::mma(accO[ct], fdb[ct & 1][kb], fp[kb]);
#pragma unroll
                for (int i = 0; i < SPW; ++i) accS[i][ct] = IO::mma(accS[i][ct], fk[i][kb], fdb[ct & 1][kb]);
            }
        }
        // o: token 16*wave + l16, columns 16*ct + 4*grp .. +3
        if constexpr (!CHK) {
            const int64_t t = (int64_t)n * kChunk + 16 * tb + l16;
            if (t < tlen && o != nullptr) {
                Tio* orow = o + ((tok0 + t) * a.H + hh) * dv + j0 + jc + 4 * grp;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) st_vec4(orow + 16 * ct, accO[ct]);
            }
        }
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int rt = tb * SPW + i;
            if (rt < SRT) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    st_vec4(&SbT[(jc + 16 * ct + l16) * SRS + 16 * rt + 4 * grp], accS[i][ct]);
                    if constexpr (CKL)
                        st_vec4(&SN[(16 * rt + 4 * grp + (l16 & 3)) * SP + jc + 16 * ct + (l16 & ~3)], quad_transpose4(accS[i][ct]));
                }
            }
        }
        __syncthreads();                                  // barrier 2
        if (NB == 1) __syncthreads();                     // barrier 3: buffer refilled
    }

    if (a.S_out != nullptr) {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int rt = tb * SPW + i;
            if (rt < SRT) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        a.S_out[(chain * DK + 16 * rt + 4 * grp + e) * dv + j0 + jc + 16 * ct + l16] = accS[i][ct][e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int chunk_state_slice(int64_t nchains, int dv, int dk, int esize)
{
    // widest slice that still gives every CU a workgroup and fits in LDS:
    // wider slices copy each chunk's factors into fewer workgroups.  When no
    // width fills the chip (few long chains), the narrowest: a chunk's
    // latency in the serial loop barely depends on the width, its work does
    // (B1 H16 T65536 d128: 16 columns 1216 us, 32 columns 1389 us)
    static const int widths[3] = {64, 32, 16};
    for (int i = 0; i < 3; ++i) {
        const int w = widths[i];
        if (dv % w == 0 && nchains * (dv / w) >= 256 && state_lds_bytes(dk, w, esize) > 0) return w;
    }
    for (int i = 2; i >= 1; --i)
        if (dv % widths[i] == 0 && state_lds_bytes(dk, widths[i], esize) > 0) return widths[i];
    return 16;
}

template <typename Tio, int DK, typename Tg>
static hipError_t prep_dk(const PrepArgs& a, hipStream_t s)
{
    const int64_t nblk = a.plan == nullptr ? a.B * a.H * (int64_t)a.nt : a.H * a.ncmax;
    if (a.t_off != 0) {                          // backward layout (bf16 I/O, dk >= 32, dv <= 128)
        if constexpr (sizeof(Tio) == 2 && DK % 32 == 0) {
            if (a.dv > 128) return hipErrorInvalidValue;
            hipLaunchKernelGGL((k_chunk_prep<Tio, DK, 8, Tg, true>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;
        }
    }
    if (a.conv_w != nullptr) {                   // fused short convolution (equal-length batches)
        if (a.plan != nullptr || a.conv_K < 1 || a.conv_K > 4) return hipErrorInvalidValue;
        if (a.dv <= 64)
            hipLaunchKernelGGL((k_chunk_prep<Tio, DK, 4, Tg, false, true>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
        else if (a.dv <= 128)
            hipLaunchKernelGGL((k_chunk_prep<Tio, DK, 8, Tg, false, true>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((k_chunk_prep<Tio, DK, 16, Tg, false, true>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
        return hipGetLastError();
    }
    if (a.dv <= 64)
        hipLaunchKernelGGL((k_chunk_prep<Tio, DK, 4, Tg>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
    else if (a.dv <= 128)
        hipLaunchKernelGGL((k_chunk_prep<Tio, DK, 8, Tg>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((k_chunk_prep<Tio, DK, 16, Tg>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename Tio, typename Tg>
static hipError_t prep_t(const PrepArgs& a, int dk, hipStream_t s)
{
    switch (dk) {
        case 16: return prep_dk<Tio, 16, Tg>(a, s);
        case 32: return prep_dk<Tio, 32, Tg>(a, s);
        case 64: return prep_dk<Tio, 64, Tg>(a, s);
        case 128: return prep_dk<Tio, 128, Tg>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_prep(const PrepArgs& a, int dk, bool bf16, bool gbf16, hipStream_t s)
{
    if (!bf16) return gbf16 ? hipErrorInvalidValue : prep_t<float, float>(a, dk, s);
    return gbf16 ? prep_t<__bf16, __bf16>(a, dk, s) : prep_t<__bf16, float>(a, dk, s);
}

template <typename Tio, int DK, int VS>
static hipError_t state_v(const StateArgs& a, hipStream_t s)
{
    if constexpr (!StateLds<Tio, DK, VS>::FITS) {
        return hipErrorInvalidValue;
    } else {
        const int64_t nblk = a.B * a.H * (int64_t)a.nslices;
        constexpr int nthreads = state_threads(VS, (int)sizeof(Tio));
        if ((a.S_chkT != nullptr || a.S_chkIo != nullptr) && !StateLds<Tio, DK, VS, true>::CKL) return hipErrorInvalidValue;
        if (a.S_chk != nullptr || a.S_chkT != nullptr || a.S_chkIo != nullptr)
            hipLaunchKernelGGL((k_chunk_state<Tio, DK, VS, true>), dim3((unsigned)nblk), dim3(nthreads), 0, s, a);
        else
            hipLaunchKernelGGL((k_chunk_state<Tio, DK, VS, false>), dim3((unsigned)nblk), dim3(nthreads), 0, s, a);
        return hipGetLastError();
    }
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
