// Per-chunk gradients of the chunked GDN-2 forward on the matrix cores
// (bf16 I/O, dk and dv in {32, 64, 128}), and the reverse state pass of the
// same path (k_chunk_state_bwd_mf, described where it is defined).
//
// Same gradient as k_chunk_grad (the formulas are in gdn2_backward.hip's
// header), in one launch of one workgroup (8 waves) per chunk, k_chunk_grad_mf,
// which runs two stages in turn in the same LDS:
//
// the value side (grad_val_chunk)  the value-side products on bf16 matrix cores, fp32
//   accumulation.  Operands come from the workspace blocks the recomputed
//   forward writes in the backward's layout (W, P^T, Ktil, U^T, T, Eh), from
//   the chunk checkpoints (S0 and the exit gradient dSL, each in bf16
//   [dk][dv] and transposed [dv][dk]) and from dO, v, w.  Every
//   operand is laid out with its contraction index contiguous (transposed
//   copies are made in LDS where needed; LDS rows are padded by 16 bytes), so
//   a fragment is one 16-byte read.  In order:
//     Delta = U - W S0,  dDelta = P^T dO + Ktil dSL,
//     dQh = dO S0^T, dP = mask(dO Delta^T), dKtil = Delta dSL^T,
//     dW = -dDelta S0^T, du = T^T dDelta (-> dw = du v, dv = du w),
//     dT = dDelta u^T + dW Eh^T, dEh = T^T dW, dA = mask(-(T^T dT) T^T),
//     dGamma_L = rowsum(dSL * S0);
//   dQh, dKtil, dEh, dP, dA (bf16) and dGamma_L (fp32) go to a scratch block
//   per chunk.
// the key side (grad_key_chunk)  the cumulative log decay G, the
//   contractions of dA and dP with the block-split decay ratios on bf16
//   matrix cores (row side: sum_s dA[r,s] k_s R[r,s]; column side:
//   sum_r dA[r,s] e_r R[r,s], and the same with dP and q), then per row the
//   gradients of q, k, b, and dalpha from the reverse cumulative sum of dG.
// With the prologue options (burn-gdn2 0.1.9 README, "Architecture" and
// "Configuration") both stages take the raw inputs: gates are activated
// on load (sigmoid, b x 2 in negative-eigenvalue mode), q/k rows normalised
// with lane-group reductions, and the gradients they write are those of
// the logits and of the raw q/k.
#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"
#include "gdn2_layout.hpp"

namespace gdn2 {

namespace {

typedef __bf16 bf;
using IOB = Io<__bf16>;
typedef IOB::frag bfrag;

constexpr int kMaxD = 128;
constexpr int LT = 64 + 8;                // padded row of a [.][64] bf16 array
constexpr int LD = kMaxD + 8;             // padded row of a [.][dk|dv] bf16 array (maximum)

// fragment (8 consecutive k) of row `row`, K-block kb, from a bf16 array with row stride ld
__device__ inline bfrag fr(const bf* base, int row, int64_t ld, int kb, int grp)
{
    return *reinterpret_cast<const bfrag*>(base + row * ld + kb * 32 + grp * 8);
}


// sum over the N consecutive lanes that hold one row (N a power of two <= 32)
template <int N>
__device__ __forceinline__ float lanes_sum(float x)
{
#pragma unroll
    for (int off = 1; off < N; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// 1 / sqrt(|x|^2 + eps) of a row spread over N lanes, 4 channels each
template <int N>
__device__ __forceinline__ float row_rnorm(f32x4 x)
{
    return __builtin_amdgcn_rsqf(lanes_sum<N>(x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]) + kL2normEps);
}

}  // namespace

// Key-axis items of a chunk on NTH threads: thread t holds channels
// c4 .. c4+3, c4 = 4 (t mod DK/4), of the NV = 16 DK / NTH consecutive rows
// (t div DK/4) NV + u, u < NV (the DK/4 lanes of a row are consecutive).
template <int DK, int NTH>
__device__ __forceinline__ void key_item(int u, int& r, int& c4)
{
    constexpr int CG = DK / 4, NV = 64 * CG / NTH;
    const int tid = threadIdx.x;
    r = (tid / CG) * NV + u;
    c4 = 4 * (tid % CG);
}

// G[r][c] = sum of log alpha over tokens 0..r of the chunk (alpha = 1 past its
// end), for NTH threads: logs in parallel (every load issued before the first
// use), then a scan of NTH/DK segments per channel with the segment totals
// carried through `tot` [NTH].  cld_load issues the loads, cld_scan does the
// rest (alpha given as logits: alpha = sigmoid(logit)).
template <int DK, int NTH, typename Tg>
__device__ __attribute__((always_inline)) inline void cld_load(typename GateVec<Tg>::type (&x)[64 * DK / 4 / NTH],
                                                               const Tg* alpha, int64_t row0, int64_t H, int Ln)
{
    constexpr int NV = 64 * DK / 4 / NTH;
#pragma unroll
    for (int u = 0; u < NV; ++u) {       // raw and unconditional (rows past the end clamped)
        int r, c4;
        key_item<DK, NTH>(u, r, c4);
        x[u] = *reinterpret_cast<const typename GateVec<Tg>::type*>(alpha + (row0 + (r < Ln ? r : Ln - 1) * H) * DK + c4);
    }
}

template <int DK, int NTH, typename Tg>
__device__ __attribute__((always_inline)) inline void cld_scan(float* G, float* tot,
                                                               const typename GateVec<Tg>::type (&x)[64 * DK / 4 / NTH],
                                                               int Ln, bool logits)
{
    constexpr int NV = 64 * DK / 4 / NTH;
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        int r, c4;
        key_item<DK, NTH>(u, r, c4);
        const f32x4 a = alpha_floor4(logits ? sigmoid4(widen4(x[u])) : widen4(x[u]));
        f32x4 l;
#pragma unroll
        for (int e = 0; e < 4; ++e) l[e] = r < Ln ? __logf(a[e]) : 0.f;   // alpha = 1 past the end
        *reinterpret_cast<f32x4*>(&G[r * DK + c4]) = l;
    }
    __syncthreads();
    constexpr int nseg = NTH / DK, sl = 64 / nseg;
    const int c = tid % DK, g = tid / DK;
    float run = 0.f;
#pragma unroll 8
    for (int r = g * sl; r < (g + 1) * sl; ++r) {
        run += G[r * DK + c];
        G[r * DK + c] = run;
    }
    tot[g * DK + c] = run;
    __syncthreads();
    float carry = 0.f;
    for (int h = 0; h < g; ++h) carry += tot[h * DK + c];
    if (g > 0)
        for (int r = g * sl; r < (g + 1) * sl; ++r) G[r * DK + c] += carry;
    __syncthreads();
}

// LDS regions of the value side (bytes), sized for dk = dv = 128
struct GvLds {
    static constexpr int R0 = 0;                                  // T [64][LT], T^T [64][LT]
    static constexpr int R1 = R0 + 2 * 64 * LT * 2;               // dO [64][LD] | u [64][LD] | tmp [64][LT]
    static constexpr int R2 = R1 + 64 * LD * 2;                   // dO^T [dv][LT] | dW [64][LD]
    static constexpr int R3 = R2 + kMaxD * LT * 2;                // P^T [64][LT] + Ktil [64][LD] | dW^T [dk][LT] + dT^T [64][LT]
    static constexpr int R3SZ = (64 * LT + 64 * LD) * 2 > (kMaxD * LT + 64 * LT) * 2 ? (64 * LT + 64 * LD) * 2
                                                                                       : (kMaxD * LT + 64 * LT) * 2;
    static constexpr int R4 = R3 + R3SZ;                          // U, then Delta [64][LD]
    static constexpr int R5 = R4 + 64 * LD * 2;                   // dDelta [64][LD] + dDelta^T [dv][LT]
    static constexpr int R7 = R5 + (64 * LD + kMaxD * LT) * 2;    // Eh [64][LD]
    static constexpr int BYTES = R7 + 64 * LD * 2;
};

constexpr int kGvThreads = 512, kGvWaves = 8;      // value-side workgroup: 8 waves

// The value side's results for the key side, handed over in LDS when both
// stages' own regions are free (bytes): dQh, dKtil, dEh bf16 [64][DK + 8],
// dP, dA bf16 [64][72], dGamma_L fp32 [DK]
template <int DK>
struct HandLds {
    static constexpr int HS = DK + 8, PS = 64 + 8;
    static constexpr int Q = 0, K = Q + 64 * HS * 2, E = K + 64 * HS * 2, P = E + 64 * HS * 2;
    static constexpr int A = P + 64 * PS * 2, GL = A + 64 * PS * 2, BYTES = GL + DK * 4;
};

// Tiles t = wave, wave + 8, ... < NT of one product: fetch(t, a, b) loads the
// NKB K-blocks of a tile's A and B fragments, epi(t, acc) consumes its
// result.  The next tile's fragments are requested before the current
// tile's products, so global-memory operands arrive while the matrix cores work.
template <int NKB, typename FF, typename FE>
__device__ __attribute__((always_inline)) inline void tiles(int wave, int NT, FF fetch, FE epi)
{
    bfrag ca[NKB], cb[NKB], na[NKB], nb[NKB];
    int t = wave;
    if (t < NT) fetch(t, na, nb);
    for (; t < NT; t += kGvWaves) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            ca[kb] = na[kb];
            cb[kb] = nb[kb];
        }
        if (t + kGvWaves < NT) fetch(t + kGvWaves, na, nb);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) acc = IOB::mma(acc, ca[kb], cb[kb]);
        epi(t, acc);
    }
}

// Column panels p = wave, wave + 8, ... < NP of products whose B operand
// (NKB K-blocks of one 16-column panel) comes from global memory: panel
// p = wave has been requested into `first`, fetch(p, b) loads a later one,
// body(p, b) runs the panel's row tiles with A from LDS.  The next panel's B
// is requested before the current panel's products.
template <int NKB, typename FF, typename FB>
__device__ __attribute__((always_inline)) inline void panels_from(int wave, int NP, const bfrag (&first)[NKB], FF fetch,
                                                                  FB body)
{
    bfrag cb[NKB], nb[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) nb[kb] = first[kb];
    for (int p = wave; p < NP; p += kGvWaves) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) cb[kb] = nb[kb];
        if (p + kGvWaves < NP) fetch(p + kGvWaves, nb);
        body(p, cb);
    }
}

template <int DK, int DV, typename Tg>
__device__ __attribute__((always_inline)) inline void grad_val_chunk(const GradVArgs& a, char* sm)
{
    using L = GvLds;
    constexpr int NTH = kGvThreads, NW = kGvWaves;
    static_assert(L::BYTES <= 160 * 1024, "LDS budget");
    constexpr int NKK = DK / 32, NKV = DV / 32, NTK = DK / 16, NTV = DV / 16;
    constexpr int ldv = DV + 8, ldk = DK + 8;
    bf* Tl = reinterpret_cast<bf*>(sm + L::R0);
    bf* Ttl = Tl + 64 * LT;
    bf* dOl = reinterpret_cast<bf*>(sm + L::R1);
    bf* ul = dOl;
    bf* tmpl = dOl;
    bf* dOtl = reinterpret_cast<bf*>(sm + L::R2);
    bf* dWl = dOtl;
    bf* Ptl = reinterpret_cast<bf*>(sm + L::R3);
    bf* Ktl = Ptl + 64 * LT;
    bf* dWtl = Ptl;
    bf* dTtl = Ptl + kMaxD * LT;
    bf* Dll = reinterpret_cast<bf*>(sm + L::R4);
    bf* dDl = reinterpret_cast<bf*>(sm + L::R5);
    bf* dDtl = dDl + 64 * ldv;
    bf* Ehl = reinterpret_cast<bf*>(sm + L::R7);

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int wave = tid >> 6;
    const int64_t ci = blockIdx.x;                   // workspace block (valid: checked by the kernel)
    ChunkPos cp;
    chunk_pos(a.plan, a.ncmax, a.B, a.T, a.H, a.nt, ci, cp);
    const int64_t hh = cp.hh;
    const int Ln = cp.len;
    const int64_t H = a.H;
    const int64_t row0 = cp.tok0 * H + hh;
    constexpr WsLayout LY = ws_layout(DK, DV, 2, 32);
    const char* blk = static_cast<const char*>(a.ws) + ci * a.ws_block;
    const bf* Tg_ = reinterpret_cast<const bf*>(blk + a.t_off);         // T [64][64]
    const bf* Ptg = reinterpret_cast<const bf*>(blk + LY.p);             // P^T [64][64]
    const bf* Kng = reinterpret_cast<const bf*>(blk + bwd_ext(a.t_off, DK).kn);   // Ktil [64][dk]
    const bf* Ehg = reinterpret_cast<const bf*>(blk + bwd_ext(a.t_off, DK).eh);   // Eh [64][dk]
    const bf* Wg = reinterpret_cast<const bf*>(blk + LY.wwy);            // W [64][dk]
    const bf* Utg = reinterpret_cast<const bf*>(blk + LY.uwyt);          // U^T [dv][64]
    const bf* S0 = static_cast<const bf*>(a.S_chk) + ci * (int64_t)DK * DV;     // [dk][dv]
    const bf* S0t = static_cast<const bf*>(a.S_chkT) + ci * (int64_t)DK * DV;   // [dv][dk]
    const bf* dSL = static_cast<const bf*>(a.dSL) + ci * (int64_t)DK * DV;
    const bf* dSLt = static_cast<const bf*>(a.dSLT) + ci * (int64_t)DK * DV;
    const bf* dO = static_cast<const bf*>(a.dO);
    const bf* vg = static_cast<const bf*>(a.v);
    const Tg* wgt = static_cast<const Tg*>(a.w);
    Tg* dwg = static_cast<Tg*>(a.dw);
    bf* dvg = static_cast<bf*>(a.dv_out);
    const bool logits = (a.flags & kFlagGateLogits) != 0;

    // ---- phase 0: operands into LDS ----------------------------------------
    // Every global load of the phase is issued before the first LDS write (one
    // round of memory latency instead of one per operand).  Granule g = tid +
    // NTH m of each operand; where an operand has fewer granules than threads
    // the extra ones load a valid granule again and store nothing.
    constexpr int GK = DK * 8, GU = DV * 8, GO = 8 * DV;           // granules of Ktil / Eh, U^T, dO
    constexpr int NTP = 64 * 8 / NTH, NKT = (GK + NTH - 1) / NTH, NUT = (GU + NTH - 1) / NTH;
    constexpr int NDO = (GO + NTH - 1) / NTH;
    static_assert(64 * 8 % NTH == 0, "T and P granules");
    bfrag tq[NTP], pq[NTP], kq[NKT], eq[NKT], uq[NUT], oq[NDO];
#pragma unroll
    for (int m = 0; m < NTP; ++m) {                                 // T, P
        const int g = tid + m * NTH, r = g >> 3, c0 = (g & 7) * 8;
        tq[m] = *reinterpret_cast<const bfrag*>(Tg_ + r * 64 + c0);
        pq[m] = *reinterpret_cast<const bfrag*>(Ptg + r * 64 + c0);
    }
#pragma unroll
    for (int m = 0; m < NKT; ++m) {                                 // Ktil [r][c]
        const int g = (tid + m * NTH) % GK, r = g / (DK / 8), c0 = (g - r * (DK / 8)) * 8;
        kq[m] = *reinterpret_cast<const bfrag*>(Kng + r * DK + c0);
        eq[m] = *reinterpret_cast<const bfrag*>(Ehg + r * DK + c0);
    }
#pragma unroll
    for (int m = 0; m < NUT; ++m) {                                 // U^T [j][r]
        const int g = (tid + m * NTH) % GU, j = g >> 3, r0 = (g & 7) * 8;
        uq[m] = *reinterpret_cast<const bfrag*>(Utg + j * 64 + r0);
    }
#pragma unroll
    for (int m = 0; m < NDO; ++m) {                                 // dO (zero past the end)
        const int g = (tid + m * NTH) % GO, r = g / (DV / 8), j0 = (g - r * (DV / 8)) * 8;
        oq[m] = *reinterpret_cast<const bfrag*>(dO + (row0 + (r < Ln ? r : Ln - 1) * H) * DV + j0);
    }
    // the first products' operands (W for every row tile, this wave's first
    // panels of S0^T and dSL^T) are requested now, behind the LDS copy below
    bfrag wa[4][NKK], pan0[2 * NKK];
#pragma unroll
    for (int tr = 0; tr < 4; ++tr)
#pragma unroll
        for (int kb = 0; kb < NKK; ++kb) wa[tr][kb] = fr(Wg, 16 * tr + l16, DK, kb, grp);
    auto fetch_pan = [&](int tn, bfrag (&fb)[2 * NKK]) {
        const int tc = tn < NTV ? tn : 0;                           // (a wave without panels loads panel 0)
#pragma unroll
        for (int kb = 0; kb < NKK; ++kb) {
            fb[kb] = fr(S0t, 16 * tc + l16, DK, kb, grp);
            fb[NKK + kb] = fr(dSLt, 16 * tc + l16, DK, kb, grp);
        }
    };
    fetch_pan(wave, pan0);
#pragma unroll
    for (int m = 0; m < NTP; ++m) {                                 // T, T^T; P^T
        const int g = tid + m * NTH, r = g >> 3, c0 = (g & 7) * 8;
        *reinterpret_cast<bfrag*>(Tl + r * LT + c0) = tq[m];
        *reinterpret_cast<bfrag*>(Ptl + r * LT + c0) = pq[m];
#pragma unroll
        for (int e = 0; e < 8; ++e) Ttl[(c0 + e) * LT + r] = tq[m][e];
    }
#pragma unroll
    for (int m = 0; m < NKT; ++m) {                                 // Ktil, Eh
        if (GK % NTH == 0 || tid + m * NTH < GK) {
            const int g = tid + m * NTH, r = g / (DK / 8), c0 = (g - r * (DK / 8)) * 8;
            *reinterpret_cast<bfrag*>(Ktl + r * ldk + c0) = kq[m];
            *reinterpret_cast<bfrag*>(Ehl + r * ldk + c0) = eq[m];
        }
    }
#pragma unroll
    for (int m = 0; m < NUT; ++m) {                                 // U [r][j] from U^T [j][r]
        if (GU % NTH == 0 || tid + m * NTH < GU) {
            const int g = tid + m * NTH, j = g >> 3, r0 = (g & 7) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) Dll[(r0 + e) * ldv + j] = uq[m][e];
        }
    }
#pragma unroll
    for (int m = 0; m < NDO; ++m) {                                 // dO, dO^T (zero past the end)
        if (GO % NTH == 0 || tid + m * NTH < GO) {
            const int g = tid + m * NTH, r = g / (DV / 8), j0 = (g - r * (DV / 8)) * 8;
            if (r >= Ln) {
#pragma unroll
                for (int e = 0; e < 8; ++e) oq[m][e] = (bf)0.f;
            }
            *reinterpret_cast<bfrag*>(dOl + r * ldv + j0) = oq[m];
#pragma unroll
            for (int e = 0; e < 8; ++e) dOtl[(j0 + e) * LT + r] = oq[m][e];
        }
    }
    // dGamma_L = rowsum(dSL * S0), fp32 sums of the bf16 checkpoints (dk < 128:
    // with dk = 128 it comes from the panels below), before the first global
    // store (a load behind a store would wait for it); stored at the end.  TPR
    // threads per row, each with DV / TPR columns, all loads in flight at once
    // (threads past DK * TPR repeat a row and store nothing).
    constexpr bool FUSE_GL = NTK % NW == 0;
    constexpr int TPR0 = NTH / DK < DV / 4 ? NTH / DK : DV / 4, TPR = TPR0 < 1 ? 1 : TPR0, NCOL = DV / TPR;
    float dgl = 0.f;
    if constexpr (!FUSE_GL) {
        const int c = (tid / TPR) % DK, sub = tid % TPR;
        bf16x4 pa[NCOL / 4], pb[NCOL / 4];
#pragma unroll
        for (int m = 0; m < NCOL / 4; ++m) {
            pa[m] = *reinterpret_cast<const bf16x4*>(dSL + (int64_t)c * DV + sub * NCOL + 4 * m);
            pb[m] = *reinterpret_cast<const bf16x4*>(S0 + (int64_t)c * DV + sub * NCOL + 4 * m);
        }
        float x = 0.f;
#pragma unroll
        for (int m = 0; m < NCOL / 4; ++m) {
            const f32x4 fa = IOB::unpack4(pa[m]), fb = IOB::unpack4(pb[m]);
            x += fa[0] * fb[0] + fa[1] * fb[1] + fa[2] * fb[2] + fa[3] * fb[3];
        }
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) x += __shfl_xor(x, off, 64);
        dgl = x;
    }
    __syncthreads();

    // ---- Delta = U - W S0 (in place over U) and dDelta = P^T dO + Ktil dSL, one
    // 16-column panel of S0^T and dSL^T at a time (W for all row tiles in registers)
    panels_from<2 * NKK>(wave, NTV, pan0, fetch_pan, [&](int tn, bfrag (&fb)[2 * NKK]) {
        const int j = 16 * tn + l16;
        const bfrag o0 = fr(dOtl, j, LT, 0, grp), o1 = fr(dOtl, j, LT, 1, grp);
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
            const int r = 16 * tr + 4 * grp;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKK; ++kb) acc = IOB::mma(acc, wa[tr][kb], fb[kb]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf* d = &Dll[(r + i) * ldv + j];
                *d = (bf)((float)*d - acc[i]);
            }
            f32x4 acd = {0.f, 0.f, 0.f, 0.f};
            acd = IOB::mma(acd, fr(Ptl, 16 * tr + l16, LT, 0, grp), o0);
            acd = IOB::mma(acd, fr(Ptl, 16 * tr + l16, LT, 1, grp), o1);
#pragma unroll
            for (int kb = 0; kb < NKK; ++kb) acd = IOB::mma(acd, fr(Ktl, 16 * tr + l16, ldk, kb, grp), fb[NKK + kb]);
#pragma unroll
            for (int i = 0; i < 4; ++i) dDl[(r + i) * ldv + j] = (bf)acd[i];
            st_vec4(dDtl + j * LT + r, acd);
        }
    });
    __syncthreads();
    // ---- dQh = dO S0^T and dW = -dDelta S0^T (one pass over S0), dKtil = Delta dSL^T
    // Every B panel of this wave (bf16 rows of S0 and dSL) is requested at
    // once, before the kernel's first global store; with dk >= 64 one wave
    // holds both the S0 and the dSL panel of a row block, and dGamma_L =
    // rowsum(dSL * S0) comes from the same fragments.
    constexpr int NPW = (2 * NTK + NW - 1) / NW;                    // panels per wave
    bfrag rb[NPW][NKV];
#pragma unroll
    for (int m = 0; m < NPW; ++m) {
        const int p = (wave + NW * m) % (2 * NTK);                 // (a wave without panels loads one again)
        const bf* B = p < NTK ? S0 : dSL;
        const int tn = p < NTK ? p : p - NTK;
#pragma unroll
        for (int kb = 0; kb < NKV; ++kb) rb[m][kb] = fr(B, 16 * tn + l16, DV, kb, grp);
    }
    float glp[FUSE_GL ? NPW / 2 : 1];
    // results for the key side, held until the end of this stage: per panel
    // and row tile, 4 rows of 4 columns after a transpose inside each lane quad
    bf16x4 hqk[NPW][4];
#pragma unroll
    for (int m = 0; m < NPW; ++m) {
        const int p = wave + NW * m;
        if (p >= 2 * NTK) break;
        const int tn = p < NTK ? p : p - NTK, c = 16 * tn + l16;
        const bfrag (&fb)[NKV] = rb[m];
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
            const int r = 16 * tr + 4 * grp;
            if (p < NTK) {
                f32x4 aq = {0.f, 0.f, 0.f, 0.f}, aw = aq;
#pragma unroll
                for (int kb = 0; kb < NKV; ++kb) {
                    aq = IOB::mma(aq, fr(dOl, 16 * tr + l16, ldv, kb, grp), fb[kb]);
                    aw = IOB::mma(aw, fr(dDl, 16 * tr + l16, ldv, kb, grp), fb[kb]);
                }
                aw = -aw;
#pragma unroll
                for (int i = 0; i < 4; ++i) dWl[(r + i) * ldk + c] = (bf)aw[i];
                st_vec4(dWtl + c * LT + r, aw);
                hqk[m][tr] = IOB::pack4(quad_transpose4(aq));
            } else {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKV; ++kb) acc = IOB::mma(acc, fr(Dll, 16 * tr + l16, ldv, kb, grp), fb[kb]);
                hqk[m][tr] = IOB::pack4(quad_transpose4(acc));
            }
        }
        if constexpr (FUSE_GL) {
            if (m >= NPW / 2) {
                float x = 0.f;
#pragma unroll
                for (int kb = 0; kb < NKV; ++kb)
#pragma unroll
                    for (int e = 0; e < 8; ++e) x += (float)rb[m][kb][e] * (float)rb[m - NPW / 2][kb][e];
                x += __shfl_xor(x, 16, 64);
                x += __shfl_xor(x, 32, 64);
                glp[m - NPW / 2] = x;
            }
        }
    }
    // ---- dP = mask(dO Delta^T) -------------------------------------------------------
    constexpr int N64 = 16 / NW;                                    // 64 x 64 tiles per wave
    bf16x4 hp[N64];
#pragma unroll
    for (int m = 0; m < N64; ++m) {
        const int t = wave + NW * m, tr = t >> 2, tn = t & 3;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKV; ++kb) acc = IOB::mma(acc, fr(dOl, 16 * tr + l16, ldv, kb, grp), fr(Dll, 16 * tn + l16, ldv, kb, grp));
        const int r = 16 * tr + 4 * grp, s = 16 * tn + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = s <= r + i ? acc[i] : 0.f;
        hp[m] = IOB::pack4(quad_transpose4(acc));
    }
    // ---- du = T^T dDelta -> dw = du v, dv = du w;  u = w v ----------------------
    // A transpose inside each lane quad turns a du tile's accumulator into rows
    // of 4 consecutive columns (lane q: row 16 tr + 4 grp + q), so w and v are
    // read once, as vectors, for dw, dv and u alike.  They are requested before
    // the first product and kept in their memory dtypes until used (a
    // conversion right after the load would wait for it); rows past the end
    // are clamped on load, never stored, and give u = 0.
    constexpr int NTU = 4 * NTV / NW;                               // du tiles per wave
    static_assert(4 * NTV % NW == 0, "du tiles");
    typedef typename GateVec<Tg>::type gvec;
    gvec wx[NTU];
    bf16x4 vx[NTU], ux[NTU];
#pragma unroll
    for (int m = 0; m < NTU; ++m) {
        const int t = wave + NW * m, tr = t / NTV, tn = t - tr * NTV;
        const int r = 16 * tr + 4 * grp + (l16 & 3), j = 16 * tn + (l16 & ~3);
        const int64_t o = (row0 + (r < Ln ? r : Ln - 1) * H) * DV + j;
        wx[m] = *reinterpret_cast<const gvec*>(wgt + o);
        vx[m] = *reinterpret_cast<const bf16x4*>(vg + o);
    }
#pragma unroll
    for (int m = 0; m < NTU; ++m) {
        const int t = wave + NW * m, tr = t / NTV, tn = t - tr * NTV;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            acc = IOB::mma(acc, fr(Ttl, 16 * tr + l16, LT, kb, grp), fr(dDtl, 16 * tn + l16, LT, kb, grp));
        const f32x4 d4 = quad_transpose4(acc);                     // du[r][j .. j+3]
        const int r = 16 * tr + 4 * grp + (l16 & 3), j = 16 * tn + (l16 & ~3);
        const f32x4 w4 = widen4(wx[m]), sw = logits ? sigmoid4(w4) : w4, v4 = IOB::unpack4(vx[m]);
        if (r < Ln) {
            const int64_t o = (row0 + r * H) * DV + j;
            const f32x4 dwa = d4 * v4;                              // gradient of the activated gate
            f32x4 dw4 = dwa;
            if (logits) {
#pragma unroll
                for (int e = 0; e < 4; ++e) dw4[e] = dwa[e] * sw[e] * (1.f - sw[e]);
            }
            st_vec4(dwg + o, dw4);
            st_vec4(dvg + o, d4 * sw);
        }
        ux[m] = IOB::pack4(r < Ln ? sw * v4 : f32x4{0.f, 0.f, 0.f, 0.f});
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NTU; ++m) {                                 // u over dO (no longer read)
        const int t = wave + NW * m, tr = t / NTV, tn = t - tr * NTV;
        *reinterpret_cast<bf16x4*>(ul + (16 * tr + 4 * grp + (l16 & 3)) * ldv + 16 * tn + (l16 & ~3)) = ux[m];
    }
    __syncthreads();
    // ---- dT = dDelta u^T + dW Eh^T (stored transposed);  dEh = T^T dW ------------
    tiles<NKV + NKK>(wave, 16,
                     [&](int t, bfrag (&fa)[NKV + NKK], bfrag (&fb)[NKV + NKK]) {
                         const int tr = t >> 2, tn = t & 3;
#pragma unroll
                         for (int kb = 0; kb < NKV; ++kb) {
                             fa[kb] = fr(dDl, 16 * tr + l16, ldv, kb, grp);
                             fb[kb] = fr(ul, 16 * tn + l16, ldv, kb, grp);
                         }
#pragma unroll
                         for (int kb = 0; kb < NKK; ++kb) {
                             fa[NKV + kb] = fr(dWl, 16 * tr + l16, ldk, kb, grp);
                             fb[NKV + kb] = fr(Ehl, 16 * tn + l16, ldk, kb, grp);
                         }
                     },
                     [&](int t, f32x4 acc) {
                         st_vec4(dTtl + (16 * (t & 3) + l16) * LT + 16 * (t >> 2) + 4 * grp, acc);
                     });
    constexpr int NEH = 4 * NTK / NW;                               // dEh tiles per wave
    static_assert(4 * NTK % NW == 0, "dEh tiles");
    bf16x4 he[NEH];
#pragma unroll
    for (int m = 0; m < NEH; ++m) {
        const int t = wave + NW * m, tr = t / NTK, tn = t - tr * NTK;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc = IOB::mma(acc, fr(Ttl, 16 * tr + l16, LT, kb, grp), fr(dWtl, 16 * tn + l16, LT, kb, grp));
        he[m] = IOB::pack4(quad_transpose4(acc));
    }
    __syncthreads();
    // ---- tmp = T^T dT -------------------------------------------------------------
    tiles<2>(wave, 16,
             [&](int t, bfrag (&fa)[2], bfrag (&fb)[2]) {
#pragma unroll
                 for (int kb = 0; kb < 2; ++kb) {
                     fa[kb] = fr(Ttl, 16 * (t >> 2) + l16, LT, kb, grp);
                     fb[kb] = fr(dTtl, 16 * (t & 3) + l16, LT, kb, grp);
                 }
             },
             [&](int t, f32x4 acc) {
                 const int r = 16 * (t >> 2) + 4 * grp, j = 16 * (t & 3) + l16;
#pragma unroll
                 for (int i = 0; i < 4; ++i) tmpl[(r + i) * LT + j] = (bf)acc[i];
             });
    __syncthreads();
    // ---- dA = mask(-tmp T^T) --------------------------------------------------------
    bf16x4 ha[N64];
#pragma unroll
    for (int m = 0; m < N64; ++m) {
        const int t = wave + NW * m, tr = t >> 2, tn = t & 3;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc = IOB::mma(acc, fr(tmpl, 16 * tr + l16, LT, kb, grp), fr(Tl, 16 * tn + l16, LT, kb, grp));
        const int r = 16 * tr + 4 * grp, s = 16 * tn + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = s < r + i ? -acc[i] : 0.f;
        ha[m] = IOB::pack4(quad_transpose4(acc));
    }
    // ---- hand-over: every LDS region of this stage is free now ----------------
    __syncthreads();
    using HL = HandLds<DK>;
    constexpr int HS = HL::HS, PS = HL::PS;
    bf* hQ = reinterpret_cast<bf*>(sm + HL::Q);
    bf* hK = reinterpret_cast<bf*>(sm + HL::K);
    bf* hE = reinterpret_cast<bf*>(sm + HL::E);
    bf* hP = reinterpret_cast<bf*>(sm + HL::P);
    bf* hA = reinterpret_cast<bf*>(sm + HL::A);
    float* hG = reinterpret_cast<float*>(sm + HL::GL);
    const int rq = 4 * grp + (l16 & 3), cq = l16 & ~3;             // lane's row and column in a tile
#pragma unroll
    for (int m = 0; m < NPW; ++m) {
        const int p = wave + NW * m;
        if (p < 2 * NTK) {
            const int tn = p < NTK ? p : p - NTK;
            bf* dst = p < NTK ? hQ : hK;
#pragma unroll
            for (int tr = 0; tr < 4; ++tr)
                *reinterpret_cast<bf16x4*>(dst + (16 * tr + rq) * HS + 16 * tn + cq) = hqk[m][tr];
        }
    }
#pragma unroll
    for (int m = 0; m < NEH; ++m) {
        const int t = wave + NW * m, tr = t / NTK, tn = t - tr * NTK;
        *reinterpret_cast<bf16x4*>(hE + (16 * tr + rq) * HS + 16 * tn + cq) = he[m];
    }
#pragma unroll
    for (int m = 0; m < N64; ++m) {
        const int t = wave + NW * m, tr = t >> 2, tn = t & 3;
        *reinterpret_cast<bf16x4*>(hP + (16 * tr + rq) * PS + 16 * tn + cq) = hp[m];
        *reinterpret_cast<bf16x4*>(hA + (16 * tr + rq) * PS + 16 * tn + cq) = ha[m];
    }
    if constexpr (FUSE_GL) {
        if (grp == 0) {
#pragma unroll
            for (int i = 0; i < NPW / 2; ++i) hG[16 * (wave + NW * i) + l16] = glp[i];
        }
    } else {
        if (tid % TPR == 0 && tid < DK * TPR) hG[tid / TPR] = dgl;
    }
}

// ---------------------------------------------------------------------------
// key side: one workgroup per chunk.  The contractions of dA and dP with the
// decay ratios run on bf16 matrix cores, split at the chunk's 8-token halves,
// each referred to its token 3 (m_h = 8h + 3) as in the forward: for rows r
// in half hr and columns s in half hs,
//   exp(G_r - G_s) = exp(G_r - G_m(hr)) * exp(G_m(hr) - G_m(hs)) * exp(G_m(hs) - G_s),
// the outer factors products of at most 4 decays or their inverses, the
// middle one (<= 1 for hr >= hs) per (hr, hs, channel) scaling the fp32 sum of
// that pair of halves.
//   row side    deA[r,c] = exp(G_r - G_m(hr)) sum_hs F[c] sum_{s in hs} dA[r,s] KY[s,c]
//               (and dqP with dP),   KY[s,c] = k_s exp(G_m(hs) - G_s)
//   column side kak[s,c] = exp(G_m(hs) - G_s) sum_hr F[c] sum_{r in hr} dA[r,s] EA[r,c]
//               + the same with dP and QA,  EA = e_r exp(G_r - G_m(hr)),
//               QA = q_r exp(G_r - G_m(hr))
// Every operand is stored in LDS with its contraction index contiguous:
// dA and dP row-major and transposed, KY, EA and QA transposed ([channel]
// [token]), written element by element from registers in phase A, so that
// every fragment of the products is one 16-byte read.  Wave w owns column
// tiles w, w+8, ... for all 64 rows.  Then a per-row pass forms
// the gradients of q, k and b and dG, and dalpha is the reverse cumulative
// sum of dG.  Every phase issues its global loads before using any of them.
// ---------------------------------------------------------------------------

constexpr int kGkThreads = 512;                    // 8 waves per key-side workgroup

template <int DK>
struct GkLds {
    static constexpr int RS = DK + 4;              // row stride of the fp32 results / dG
    static constexpr int IN_A = 0;                 // dA, dP [64][LT] bf16
    static constexpr int IN_AT = IN_A + 2 * 64 * LT * 2;  // dA^T, dP^T [64][LT] bf16
    static constexpr int IN_K = IN_AT + 2 * 64 * LT * 2;  // KY^T, EA^T, QA^T [DK][LT] bf16
    static constexpr int SZ_IN = IN_K + 3 * DK * LT * 2;
    static constexpr int SZ_RES = 3 * 64 * RS * 4;        // deA (then dG), dqP, kak fp32 [64][RS]
    static constexpr int BIG = SZ_IN > SZ_RES ? SZ_IN : SZ_RES;
    // the workgroup's LDS: G fp32 [64][DK], the operands / results region, the
    // per row group column sums and the scan totals
    static constexpr int O_G = 0, O_BIG = 64 * DK * 4, O_EXT = O_BIG + BIG;
    static constexpr int O_TOT = O_EXT + (kGkThreads / (DK / 4)) * DK * 4;
    static constexpr int BYTES = O_TOT + kGkThreads * 4;
};

template <int DK, typename Tg>
__device__ __attribute__((always_inline)) inline void grad_key_chunk(const GradKArgs& a, char* sm)
{
    using L = GkLds<DK>;
    constexpr int NTH = kGkThreads, NW = NTH / 64;
    constexpr int CG = DK / 4, R = 64 * CG / NTH, NCT = DK / 16, CPW = (NCT + NW - 1) / NW;
    constexpr int RS = L::RS;
    constexpr int NV = 64 * DK / 4 / NTH;
    typedef typename GateVec<Tg>::type gvec;
    float* G = reinterpret_cast<float*>(sm + L::O_G);
    char* big = sm + L::O_BIG;
    float* ext = reinterpret_cast<float*>(sm + L::O_EXT);      // per row group: sum of dKtil * Ktil
    float* tot = reinterpret_cast<float*>(sm + L::O_TOT);
    bf* dAl = reinterpret_cast<bf*>(big + L::IN_A);
    bf* dPl = dAl + 64 * LT;
    bf* dATl = reinterpret_cast<bf*>(big + L::IN_AT);
    bf* dPTl = dATl + 64 * LT;
    bf* KYTl = reinterpret_cast<bf*>(big + L::IN_K);
    bf* EATl = KYTl + DK * LT;
    bf* QATl = EATl + DK * LT;
    float* deAl = reinterpret_cast<float*>(big);               // results, after the products
    float* dqPl = deAl + 64 * RS;
    float* kakl = dqPl + 64 * RS;
    float* dG = deAl;                                          // over deA, element by element

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int wave = tid >> 6;
    const int64_t ci = blockIdx.x;                   // workspace block (valid: checked by the kernel)
    ChunkPos cp;
    chunk_pos(a.plan, a.ncmax, a.B, a.T, a.H, a.nt, ci, cp);
    const int64_t hh = cp.hh;
    const int Ln = cp.len;
    const int64_t H = a.H;
    const int64_t row0 = cp.tok0 * H + hh;
    const bf* qg = static_cast<const bf*>(a.q);
    const bf* kg = static_cast<const bf*>(a.k);
    const Tg* agt = static_cast<const Tg*>(a.alpha);
    const Tg* bgt = static_cast<const Tg*>(a.b);
    const bool logits = (a.flags & kFlagGateLogits) != 0, l2 = (a.flags & kFlagQkL2norm) != 0;
    const float bscale = (a.flags & kFlagNegEigval) ? 2.f : 1.f;

    // ---- the value side's results, from the hand-over region of LDS -----------
    // (the row pass's dQh, dEh, dKtil at this thread's key items; dA and dP in
    // the 8 x 8 blocks of phase A; dGamma_L)
    using HL = HandLds<DK>;
    const int c0 = 4 * (tid % CG), r0 = (tid / CG) * R;
    bf16x4 xqh[R], xeh[R], xkt[R];                                 // raw until used
    bfrag xb[8];
    const int bk = tid & 63, bR = bk >> 3, bS = bk & 7;
    float dglv;
    {
        const bf* hQ = reinterpret_cast<const bf*>(sm + HL::Q);
        const bf* hK = reinterpret_cast<const bf*>(sm + HL::K);
        const bf* hE = reinterpret_cast<const bf*>(sm + HL::E);
        const bf* bsrc = reinterpret_cast<const bf*>(sm + ((tid & 64) ? HL::P : HL::A));
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int r = r0 + rr;
            xqh[rr] = *reinterpret_cast<const bf16x4*>(hQ + r * HL::HS + c0);
            xeh[rr] = *reinterpret_cast<const bf16x4*>(hE + r * HL::HS + c0);
            xkt[rr] = *reinterpret_cast<const bf16x4*>(hK + r * HL::HS + c0);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) xb[e] = *reinterpret_cast<const bfrag*>(bsrc + (8 * bR + e) * HL::PS + 8 * bS);
        dglv = reinterpret_cast<const float*>(sm + HL::GL)[tid < DK ? tid : 0];
    }
    __syncthreads();                                           // read: this stage's regions overwrite it

    // ---- phase A: loads (raw), then dA, dP, G, KY, EA, QA into LDS ----------
    // alpha, b, k, q stay in registers, raw, for the row pass and dalpha (the
    // row pass's rows are this thread's key items)
    static_assert(R == NV, "row pass on the key items");
    gvec ax[NV], bx[NV];
    bf16x4 kx[NV], qx[NV];
    {
        // dA and dP in 8 x 8 blocks: thread t < 128 holds block t mod 64 of dA
        // (t < 64) or dP, rows 8 (b / 8) .., columns 8 (b mod 8) ..; it writes
        // the block row-major and, transposed in registers, into the
        // transposed copy
        cld_load<DK, NTH>(ax, agt, row0, H, Ln);
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            int r, c4;
            key_item<DK, NTH>(u, r, c4);
            const int64_t o = (row0 + (r < Ln ? r : Ln - 1) * H) * DK + c4;
            kx[u] = *reinterpret_cast<const bf16x4*>(kg + o);
            qx[u] = *reinterpret_cast<const bf16x4*>(qg + o);
            bx[u] = *reinterpret_cast<const gvec*>(bgt + o);
        }
        if (tid < 128) {
            bf* dst = (tid & 64) ? dPl : dAl;
            bf* dstT = (tid & 64) ? dPTl : dATl;
#pragma unroll
            for (int e = 0; e < 8; ++e) *reinterpret_cast<bfrag*>(dst + (8 * bR + e) * LT + 8 * bS) = xb[e];
#pragma unroll
            for (int f = 0; f < 8; ++f) {
                bfrag y;
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = xb[e][f];
                *reinterpret_cast<bfrag*>(dstT + (8 * bS + f) * LT + 8 * bR) = y;
            }
        }
        cld_scan<DK, NTH, Tg>(G, tot, ax, Ln, logits);
        // KY, EA, QA transposed: a thread's NV consecutive rows of one channel
        // are one vector store
        typedef bf rowv __attribute__((ext_vector_type(NV)));
        rowv ty[4], te[4], tq[4];
        int rb = 0, cb = 0;
        key_item<DK, NTH>(0, rb, cb);
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            int r, c4;
            key_item<DK, NTH>(u, r, c4);
            const f32x4 g4 = *reinterpret_cast<const f32x4*>(&G[r * DK + c4]);
            const f32x4 gj = *reinterpret_cast<const f32x4*>(&G[((r & ~7) | 3) * DK + c4]);   // half's midpoint
            const bool ok = r < Ln;
            f32x4 k4 = IOB::unpack4(kx[u]), q4 = IOB::unpack4(qx[u]);
            const f32x4 b4 = logits ? sigmoid4(widen4(bx[u])) * bscale : widen4(bx[u]);
            if (l2) {
                k4 = k4 * row_rnorm<CG>(k4);
                q4 = q4 * row_rnorm<CG>(q4);
            }
            f32x4 ky, ea, qa;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float up = __expf(g4[e] - gj[e]);        // a product of at most 4 decays or its inverse
                ky[e] = ok ? k4[e] * __expf(gj[e] - g4[e]) : 0.f;
                ea[e] = ok ? b4[e] * k4[e] * up : 0.f;
                qa[e] = ok ? q4[e] * up : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ty[e][u] = (bf)ky[e];
                te[e][u] = (bf)ea[e];
                tq[e][u] = (bf)qa[e];
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            *reinterpret_cast<rowv*>(KYTl + (cb + e) * LT + rb) = ty[e];
            *reinterpret_cast<rowv*>(EATl + (cb + e) * LT + rb) = te[e];
            *reinterpret_cast<rowv*>(QATl + (cb + e) * LT + rb) = tq[e];
        }
    }
    __syncthreads();

    // ---- products on the matrix cores: column tiles ct = wave + NW m ---------
    f32x4 acc[CPW][4][4];                                      // [tile][row block][rowA rowP colA colP]
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
        const int ct = wave + NW * m;
        const int c = 16 * (ct < NCT ? ct : 0) + l16;
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) acc[m][I][qd] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (ct >= NCT) continue;
            // One product per pair of 8-token halves: the A operand keeps only
            // the lanes whose 8 tokens form the other half (a K-block holds
            // four), and the decay between the two halves' reference tokens
            // (token 3 of each half; <= 1) scales the fp32 sum.  With KY, EA,
            // QA referred to their own half's reference token, every factor
            // stays within a product of 4 decays or its inverse, and every pair
            // term dA[r][s] KY_s EA_r enters the row sums and the column sums
            // with the same bf16 factors, which lets them cancel in dlog(alpha)
            // (below) down to fp32 rounding.  A lane's accumulator rows
            // 4 grp .. 4 grp + 3 lie in half 2 I + grp / 2 of the tile's rows.
            const int hown = 2 * I + (grp >> 1);
            const float gown = G[(8 * hown + 3) * DK + c];
            // row side: source halves 0 .. 2I+1 (dA, dP are zero for s >= r)
#pragma unroll
            for (int hs = 0; hs <= 2 * I + 1; ++hs) {
                const int kb = hs >> 2;
                const bool mine = grp == (hs & 3);
                const bfrag bk = fr(KYTl, c, LT, kb, grp);
                f32x4 ta = {0.f, 0.f, 0.f, 0.f}, tp = ta;
                ta = IOB::mma(ta, keep_or_zero(fr(dAl, 16 * I + l16, LT, kb, grp), mine), bk);
                tp = IOB::mma(tp, keep_or_zero(fr(dPl, 16 * I + l16, LT, kb, grp), mine), bk);
                const float f = hs <= hown ? __expf(gown - G[(8 * hs + 3) * DK + c]) : 0.f;   // 0: above the diagonal
                acc[m][I][0] += f * ta;
                acc[m][I][1] += f * tp;
            }
            // column side: r over halves 2I .. 7 (dA[r][s] is zero for r <= s)
#pragma unroll
            for (int hr = 2 * I; hr < 8; ++hr) {
                const int kb = hr >> 2;
                const bool mine = grp == (hr & 3);
                const int s = 16 * I + l16;
                f32x4 ta = {0.f, 0.f, 0.f, 0.f}, tp = ta;
                ta = IOB::mma(ta, keep_or_zero(fr(dATl, s, LT, kb, grp), mine), fr(EATl, c, LT, kb, grp));
                tp = IOB::mma(tp, keep_or_zero(fr(dPTl, s, LT, kb, grp), mine), fr(QATl, c, LT, kb, grp));
                const float f = hr >= hown ? __expf(G[(8 * hr + 3) * DK + c] - gown) : 0.f;
                acc[m][I][2] += f * ta;
                acc[m][I][3] += f * tp;
            }
        }
    }
    __syncthreads();                                           // inputs read; results overwrite them
#pragma unroll
    for (int m = 0; m < CPW; ++m) {
        const int ct = wave + NW * m;
        if (ct >= NCT) continue;
        const int c = 16 * ct + l16;
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // the sums before their row factors (the per-row pass applies them)
                const int r = 16 * I + 4 * grp + i;
                deAl[r * RS + c] = acc[m][I][0][i];
                dqPl[r * RS + c] = acc[m][I][1][i];
                kakl[r * RS + c] = acc[m][I][2][i] + acc[m][I][3][i];
            }
        }
    }
    __syncthreads();

    // ---- per row: the gradients of q, k, b and dG ------------------------------
    {
        bf* dq = static_cast<bf*>(a.dq);
        bf* dk_out = static_cast<bf*>(a.dk_out);
        Tg* db = static_cast<Tg*>(a.db);
        float ex[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int r = r0 + rr;
            const bool ok = r < Ln;
            const f32x4 dQh = IOB::unpack4(xqh[rr]), dEh = IOB::unpack4(xeh[rr]), dKt = IOB::unpack4(xkt[rr]);
            f32x4 q4 = IOB::unpack4(qx[rr]), k4 = IOB::unpack4(kx[rr]);
            const f32x4 braw = widen4(bx[rr]);
            const f32x4 sb = logits ? sigmoid4(braw) : braw, b4 = logits ? sb * bscale : braw;
            float nq = 1.f, nk = 1.f;                                 // 1 / norms with the L2 option
            if (l2) {
                nq = row_rnorm<CG>(q4);
                nk = row_rnorm<CG>(k4);
                q4 = q4 * nq;
                k4 = k4 * nk;
            }
            const f32x4 sA = *reinterpret_cast<const f32x4*>(&deAl[r * RS + c0]);
            const f32x4 sP = *reinterpret_cast<const f32x4*>(&dqPl[r * RS + c0]);
            const f32x4 sC = *reinterpret_cast<const f32x4*>(&kakl[r * RS + c0]);
            f32x4 oq, okk, ob, dg;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const int c = c0 + cc;
                const float g = G[r * DK + c], gam = __expf(g), kt = __expf(G[63 * DK + c] - g);
                const float gI = G[((r & ~7) | 3) * DK + c];            // the half's reference token
                const float xr = __expf(g - gI), y = __expf(gI - g);   // as phase A forms EA, QA, KY
                const float qv = ok ? q4[cc] : 0.f, kv = ok ? k4[cc] : 0.f, bv = ok ? b4[cc] : 0.f, ev = bv * kv;
                const float deA = sA[cc] * xr, dqP = sP[cc] * xr, kak = sC[cc] * y;
                const float de = gam * dEh[cc] + deA;
                oq[cc] = gam * dQh[cc] + dqP;
                okk[cc] = kt * dKt[cc] + de * bv + kak;
                ob[cc] = de * kv;
                // the pair terms of A and P with the bf16 EA, QA, KY the products
                // used, so that the pairs of dG inside [t, 64) cancel in the
                // reverse sum below
                const float eab = (float)(bf)(ev * xr), qab = (float)(bf)(qv * xr), kyb = (float)(bf)(kv * y);
                dg[cc] = dQh[cc] * gam * qv + dEh[cc] * gam * ev - dKt[cc] * kv * kt + sA[cc] * eab +
                         sP[cc] * qab - sC[cc] * kyb;
                ex[cc] += dKt[cc] * kv * kt;
            }
            *reinterpret_cast<f32x4*>(&dG[r * RS + c0]) = dg;
            if (l2) {   // through the norms: dx = (dxh - xh (xh . dxh)) / |x|
                const f32x4 qh = ok ? q4 : f32x4{0.f, 0.f, 0.f, 0.f}, kh = ok ? k4 : f32x4{0.f, 0.f, 0.f, 0.f};
                const float sq = lanes_sum<CG>(qh[0] * oq[0] + qh[1] * oq[1] + qh[2] * oq[2] + qh[3] * oq[3]);
                const float sk = lanes_sum<CG>(kh[0] * okk[0] + kh[1] * okk[1] + kh[2] * okk[2] + kh[3] * okk[3]);
                oq = (oq - qh * sq) * nq;
                okk = (okk - kh * sk) * nk;
            }
            if (logits) ob = ob * (sb * (1.f - sb)) * bscale;            // gradient of the logit
            if (ok) {
                const int64_t o = (row0 + r * H) * DK + c0;
                st_vec4(dq + o, oq);
                st_vec4(dk_out + o, okk);
                st_vec4(db + o, ob);
            }
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) ext[(tid / CG) * DK + c0 + cc] = ex[cc];
    }
    __syncthreads();
    // dlog(alpha) = reverse cumulative sum of dG; the last token also carries
    // the uses of Gamma_L (the state decay over the chunk and Ktil)
    if (tid < DK) {
        float x = dglv * __expf(G[63 * DK + tid]);
        for (int g = 0; g < NTH / CG; ++g) x += ext[g * DK + tid];
        dG[63 * RS + tid] += x;
    }
    __syncthreads();
    {
        const int nseg = NTH / DK, sl = 64 / nseg;
        const int c = tid % DK, g = tid / DK;
        float run = 0.f;
        for (int r = (g + 1) * sl - 1; r >= g * sl; --r) {
            run += dG[r * RS + c];
            dG[r * RS + c] = run;
        }
        tot[g * DK + c] = run;
        __syncthreads();
        float carry = 0.f;
        for (int h = g + 1; h < nseg; ++h) carry += tot[h * DK + c];
        if (g + 1 < nseg)
            for (int r = g * sl; r < (g + 1) * sl; ++r) dG[r * RS + c] += carry;
    }
    __syncthreads();
    {
        Tg* dalpha = static_cast<Tg*>(a.dalpha);
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            int r, c4;
            key_item<DK, NTH>(u, r, c4);
            if (r < Ln) {
                const int64_t o = (row0 + r * H) * DK + c4;
                const f32x4 a4 = widen4(ax[u]), g4 = *reinterpret_cast<const f32x4*>(&dG[r * RS + c4]);
                f32x4 d4;
                // a decay below the floor was raised to it: the forward does not
                // depend on it there, and its gradient is 0
                if (logits) {   // d logit = (dG / alpha) alpha (1 - alpha), alpha = sigmoid(logit)
                    const f32x4 s4 = sigmoid4(a4);
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc) d4[cc] = s4[cc] < kAlphaFloor ? 0.f : g4[cc] * (1.f - s4[cc]);
                } else {
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc) d4[cc] = a4[cc] < kAlphaFloor ? 0.f : g4[cc] / a4[cc];
                }
                st_vec4(dalpha + o, d4);
            }
        }
    }
}

// One workgroup per chunk runs the value side, then the key side of the same
// chunk in the same LDS; the value side's results pass from one to the other
// through LDS (HandLds), written when the value side's regions are free and
// read before the key side's overwrite them.
template <int DK, int DV, typename Tg>
__global__ __launch_bounds__(kGvThreads, 1) void k_chunk_grad_mf(GradVArgs v, GradKArgs k)
{
    static_assert(kGvThreads == kGkThreads, "one workgroup shape for both sides");
    constexpr int B0 = GvLds::BYTES > GkLds<DK>::BYTES ? GvLds::BYTES : GkLds<DK>::BYTES;
    constexpr int BYTES = B0 > HandLds<DK>::BYTES ? B0 : HandLds<DK>::BYTES;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) char sm[BYTES];
    ChunkPos cp;
    if (!chunk_pos(v.plan, v.ncmax, v.B, v.T, v.H, v.nt, blockIdx.x, cp)) return;   // past a packed batch's chunks
    grad_val_chunk<DK, DV, Tg>(v, sm);
    __syncthreads();                       // the hand-over written
    grad_key_chunk<DK, Tg>(k, sm);
}

// ---------------------------------------------------------------------------
// Reverse state pass of the matrix-core path: one workgroup per (batch, head,
// 32-column slice), 4 compute waves and 8 loader waves, chunks in reverse.
// The gradient dS [dk][32] of the chunk's exit state lives in the compute
// waves' accumulators (wave w: row tiles w, w + 4, ...).  Per chunk:
//   dDelta = P^T dO + Ktil dS                  (wave w: rows 16w .. 16w+15)
//                                                            | barrier 1
//   dS     = diag(Gamma_L) dS + Qh^T dO - W^T dDelta         | barrier 2
// The factors come in the backward's layout of the workspace block (Qh^T,
// P^T, Ktil, W^T: contraction index contiguous), so every A fragment is one
// 16-byte LDS read; the B operands dO, dS (bf16) and dDelta are kept
// transposed in LDS.  Loader waves keep the next chunks' factors and dO in
// flight in their registers and copy chunk n-1 into the second LDS buffer
// (half before barrier 1, half after) while chunk n is computed, dO
// transposed on the way.  The exit gradient of each chunk is written in bf16,
// [dk][dv] and transposed [dv][dk]: the compute waves keep both layouts in
// LDS (dS^T is their operand anyway) and the loader waves copy them out
// before barrier 1, so that no global store sits in the compute waves' path.
// The slices of one head get block ids congruent mod 8 (one XCD, one L2 for
// the head's blocks).
// ---------------------------------------------------------------------------
template <int DK>
struct RsLds {
    static constexpr int VS = 32;                      // value columns per workgroup
    static constexpr int RP = 64 + 8;                  // padded row of a [.][64] bf16 array
    static constexpr int KR = DK + 8;                  // padded row of a [.][DK] bf16 array
    // one operand buffer
    static constexpr int QT = 0;                       // Qh^T [DK][RP]
    static constexpr int PT = QT + DK * RP * 2;        // P^T [64][RP]
    static constexpr int WT = PT + 64 * RP * 2;        // W^T [DK][RP]
    static constexpr int KN = WT + DK * RP * 2;        // Ktil [64][KR]
    static constexpr int GL = KN + 64 * KR * 2;        // Gamma_L fp32 [DK]
    static constexpr int OT = GL + DK * 4;             // dO^T [VS][RP]
    static constexpr int BUF = OT + VS * RP * 2;
    static constexpr int DT = 2 * BUF;                 // dDelta^T [VS][RP]
    static constexpr int ST = DT + VS * RP * 2;        // dS^T bf16 [VS][KR]
    static constexpr int SP = VS + 8;                  // padded row of dS
    static constexpr int SN = ST + VS * KR * 2;        // dS bf16 [DK][SP]
    static constexpr int BYTES = SN + DK * SP * 2;
    static constexpr int G_CK = VS * DK / 8;           // granules of one layout of the exit gradient
    // 16-byte granules of one chunk: dO (64 rows of VS columns), then Qh^T,
    // P^T, W^T, Ktil, Gamma_L
    static constexpr int G_DO = 64 * VS / 8;
    static constexpr int G_QT = DK * 8, G_PT = 64 * 8, G_WT = DK * 8, G_KN = 64 * DK / 8, G_GL = DK / 4;
    static constexpr int NG = G_DO + G_QT + G_PT + G_WT + G_KN + G_GL;
    static constexpr int NCW = 4, NLW = 8;             // compute and loader waves
    static constexpr int NLD = 64 * NLW;
    static constexpr int LPL = (NG + NLD - 1) / NLD;   // granules per loader lane per chunk
    static constexpr int THREADS = 64 * (NCW + NLW);
};

template <int DK>
__global__ __launch_bounds__(RsLds<DK>::THREADS, 1) void k_chunk_state_bwd_mf(BwdStateArgs a)
{
    using L = RsLds<DK>;
    constexpr int RP = L::RP, KR = L::KR, VS = L::VS, LPL = L::LPL, NCW = L::NCW;
    constexpr int NTC = DK / 16, TPW = (NTC + 3) / 4, NKK = DK / 32;
    constexpr WsLayout LY = ws_layout(DK, 0, 2, 32);
    static_assert(L::G_DO == 4 * 64 && L::BYTES <= 160 * 1024, "layout");
    __shared__ __attribute__((aligned(16))) char sm[L::BYTES];
    bf* DTl = reinterpret_cast<bf*>(sm + L::DT);
    bf* STl = reinterpret_cast<bf*>(sm + L::ST);
    bf* SNl = reinterpret_cast<bf*>(sm + L::SN);

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int dv = a.dv;
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
    // the sequence's tokens, chunk count and first block
    const ChainSpan sp = chain_span(a.plan, a.ncmax, a.B, a.T, a.H, a.nt, bb, hh);
    const int nt = sp.nt;

    if (wave >= NCW) {
        // ---------------- loader waves ------------------------------------
        // Step i of the pass works on chunk nt-1-i; its operands go to buffer
        // i & 1.  Granule g = (wave - NCW)*64 + lane + NLD*m: slot 0 of loader
        // waves 0..3 holds dO (row g/4, columns 8(g%4) .. +7 of the slice);
        // every other slot a factor granule (source offset in the block,
        // destination in the buffer); idle slots copy a factor granule some
        // other lane copies too (the same bytes to the same place).
        const int lw = wave - NCW;
        const bool dol = lw < 4;
        const bf* dO = static_cast<const bf*>(a.dO);
        const int dr = (lw * 64 + lane) >> 2, dc = 8 * (lane & 3);
        int src[LPL], dst[LPL];
#pragma unroll
        for (int m = 0; m < LPL; ++m) {
            int g = lw * 64 + lane + L::NLD * m - L::G_DO;
            if (g >= L::NG - L::G_DO) g %= (L::NG - L::G_DO);
            if (g < 0) g = 0;                                // (dO slot: unused)
            const BwdExt X = bwd_ext(a.t_off, DK);
            int sr, ds;
            if (g < L::G_QT) {
                sr = (int)LY.qh + 16 * g;
                ds = L::QT + (g >> 3) * RP * 2 + (g & 7) * 16;
            } else if ((g -= L::G_QT) < L::G_PT) {
                sr = (int)LY.p + 16 * g;
                ds = L::PT + (g >> 3) * RP * 2 + (g & 7) * 16;
            } else if ((g -= L::G_PT) < L::G_WT) {
                sr = (int)X.wt + 16 * g;
                ds = L::WT + (g >> 3) * RP * 2 + (g & 7) * 16;
            } else if ((g -= L::G_WT) < L::G_KN) {
                sr = (int)X.kn + 16 * g;
                ds = L::KN + (g / (DK / 8)) * KR * 2 + (g % (DK / 8)) * 16;
            } else {
                g -= L::G_KN;
                sr = (int)LY.gaml + 16 * g;
                ds = L::GL + 16 * g;
            }
            src[m] = sr;
            dst[m] = ds;
        }
        // register slots of chunks in flight: as many as fit, without spills,
        // in the 168 registers of three waves per SIMD (dk = 128: two)
        constexpr int DEPTH0 = (168 - 2 * LPL - 80) / (4 * LPL);
        constexpr int DEPTH = DEPTH0 > 4 ? 4 : (DEPTH0 < 1 ? 1 : DEPTH0);
        bfrag r[DEPTH][LPL];
        // granules [m0, m1) of step i into / out of a register slot; steps past
        // the end load chunk 0 again (every step issues the same loads)
        auto fetch = [&](int i, bfrag* rs, int m0, int m1) {
            const int n = nt - 1 - i < 0 ? 0 : nt - 1 - i;
            const char* blk = static_cast<const char*>(a.ws) + (sp.blk0 + n) * a.ws_block;
            const int64_t t0 = (int64_t)n * kChunk;
            const int Ln = (int)(sp.tlen - t0 < kChunk ? sp.tlen - t0 : kChunk);
            const int rc = dr < Ln ? dr : Ln - 1;
            const char* pd = reinterpret_cast<const char*>(dO + ((sp.tok0 + t0 + rc) * a.H + hh) * dv + j0 + dc);
#pragma unroll
            for (int m = 0; m < LPL; ++m)
                if (m >= m0 && m < m1)
                    rs[m] = *reinterpret_cast<const bfrag*>(m == 0 && dol ? pd : blk + src[m]);
        };
        auto store = [&](int i, const bfrag* rs, int m0, int m1) {
            char* b0 = sm + (i & 1) * L::BUF;
#pragma unroll
            for (int m = 0; m < LPL; ++m) {
                if (m >= m0 && m < m1) {
                    if (m == 0 && dol) {                    // dO^T, zero past the end
                        const int n = nt - 1 - i < 0 ? 0 : nt - 1 - i;
                        const int64_t t0 = (int64_t)n * kChunk;
                        const int Ln = (int)(sp.tlen - t0 < kChunk ? sp.tlen - t0 : kChunk);
                        bf* ot = reinterpret_cast<bf*>(b0 + L::OT);
#pragma unroll
                        for (int e = 0; e < 8; ++e) ot[(dc + e) * RP + dr] = dr < Ln ? rs[0][e] : (bf)0.f;
                    } else {
                        *reinterpret_cast<bfrag*>(b0 + dst[m]) = rs[m];
                    }
                }
            }
        };
        // the exit gradient of step i's chunk from LDS to both global layouts
        // (dS^T rows [dv][dk], dS rows [dk][dv]): granule q < G_CK of dS^T,
        // then of dS
        auto ckpt = [&](int i) {
            const int64_t cb = (sp.blk0 + (nt - 1 - i)) * (int64_t)DK * dv;
#pragma unroll
            for (int q0 = 0; q0 < 2 * L::G_CK; q0 += L::NLD) {
                const int q = q0 + lw * 64 + lane;
                if (q < L::G_CK) {
                    const int j = q / (DK / 8), c8 = 8 * (q % (DK / 8));
                    const bfrag v = *reinterpret_cast<const bfrag*>(STl + j * KR + c8);
                    if (a.dSLT != nullptr) *reinterpret_cast<bfrag*>(static_cast<bf*>(a.dSLT) + cb + (int64_t)(j0 + j) * DK + c8) = v;
                } else if (q < 2 * L::G_CK) {
                    const int c = (q - L::G_CK) / (VS / 8), j8 = 8 * ((q - L::G_CK) % (VS / 8));
                    const bfrag v = *reinterpret_cast<const bfrag*>(SNl + c * L::SP + j8);
                    if (a.dSLIo != nullptr) *reinterpret_cast<bfrag*>(static_cast<bf*>(a.dSLIo) + cb + (int64_t)c * dv + j0 + j8) = v;
                }
            }
        };
        // Step i: the exit gradient of step i's chunk goes out, step i+1 goes
        // to LDS and step i+1+DEPTH is requested into the slot it leaves, half
        // before barrier 1 and half after it.
        constexpr int HALF = LPL / 2 > 0 ? LPL / 2 : 1;
        auto iter = [&](int i, bfrag* rs) {
            ckpt(i);
            store(i + 1, rs, 0, HALF);
            fetch(i + 1 + DEPTH, rs, 0, HALF);
            __syncthreads();                                  // barrier 1
            store(i + 1, rs, HALF, LPL);
            fetch(i + 1 + DEPTH, rs, HALF, LPL);
            __syncthreads();                                  // barrier 2
        };
        if (nt == 0) {
            __syncthreads();                                  // prologue barrier
            return;
        }
        fetch(0, r[0], 0, LPL);
        if (DEPTH > 1) fetch(1, r[DEPTH > 1 ? 1 : 0], 0, LPL);
        store(0, r[0], 0, LPL);
        __syncthreads();                                      // prologue barrier
#pragma unroll
        for (int d = 2; d < DEPTH; ++d) fetch(d, r[d], 0, LPL);
        fetch(DEPTH, r[0], 0, LPL);
        int i = 0;
        for (; i + DEPTH <= nt; i += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) iter(i + d, r[(d + 1) % DEPTH]);
        }
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d)
            if (i + d < nt) iter(i + d, r[(d + 1) % DEPTH]);
        return;
    }

    // ---------------- compute waves -------------------------------------------
    // dS: lane (l16, grp) of tile (t, ct) holds dS[16 tc + 4 grp + e][j0 + 16 ct + l16], tc = wave + 4t
    f32x4 accS[TPW][2];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int tc = wave + 4 * t;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (tc < NTC && a.dS_T != nullptr) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = a.dS_T[(chain * DK + 16 * tc + 4 * grp + e) * dv + j0 + 16 * ct + l16];
            }
            accS[t][ct] = v;
            if (tc < NTC) {
                st_vec4(STl + (16 * ct + l16) * KR + 16 * tc + 4 * grp, v);
                st_vec4(SNl + (16 * tc + 4 * grp + (l16 & 3)) * L::SP + 16 * ct + (l16 & ~3), quad_transpose4(v));
            }
        }
    }
    __syncthreads();                                          // prologue barrier
    for (int i = 0; i < nt; ++i) {
        const char* B0 = sm + (i & 1) * L::BUF;
        const bf* QTl = reinterpret_cast<const bf*>(B0 + L::QT);
        const bf* PTl = reinterpret_cast<const bf*>(B0 + L::PT);
        const bf* WTl = reinterpret_cast<const bf*>(B0 + L::WT);
        const bf* KNl = reinterpret_cast<const bf*>(B0 + L::KN);
        const float* GLl = reinterpret_cast<const float*>(B0 + L::GL);
        const bf* OTl = reinterpret_cast<const bf*>(B0 + L::OT);
        // dDelta rows 16 wave .. +15 -> dDelta^T
        {
            bfrag pa[2], ka[NKK];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) pa[kb] = fr(PTl, 16 * wave + l16, RP, kb, grp);
#pragma unroll
            for (int kb = 0; kb < NKK; ++kb) ka[kb] = fr(KNl, 16 * wave + l16, KR, kb, grp);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) acc = IOB::mma(acc, pa[kb], fr(OTl, 16 * ct + l16, RP, kb, grp));
#pragma unroll
                for (int kb = 0; kb < NKK; ++kb) acc = IOB::mma(acc, ka[kb], fr(STl, 16 * ct + l16, KR, kb, grp));
                st_vec4(DTl + (16 * ct + l16) * RP + 16 * wave + 4 * grp, acc);
            }
        }
        __syncthreads();                                      // barrier 1
        // dS = diag(Gamma_L) dS + Qh^T dO - W^T dDelta -> dS^T for the next chunk
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int tc = wave + 4 * t;
            if (tc < NTC) {
                bfrag qa[2], wa[2];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    qa[kb] = fr(QTl, 16 * tc + l16, RP, kb, grp);
                    wa[kb] = fr(WTl, 16 * tc + l16, RP, kb, grp);
                }
                const f32x4 gl = *reinterpret_cast<const f32x4*>(GLl + 16 * tc + 4 * grp);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        a1 = IOB::mma(a1, qa[kb], fr(OTl, 16 * ct + l16, RP, kb, grp));
                        a2 = IOB::mma(a2, wa[kb], fr(DTl, 16 * ct + l16, RP, kb, grp));
                    }
                    accS[t][ct] = gl * accS[t][ct] + a1 - a2;
                    // dS^T and dS (lane q of a quad: row 16 tc + 4 grp + q) for the next chunk
                    st_vec4(STl + (16 * ct + l16) * KR + 16 * tc + 4 * grp, accS[t][ct]);
                    st_vec4(SNl + (16 * tc + 4 * grp + (l16 & 3)) * L::SP + 16 * ct + (l16 & ~3), quad_transpose4(accS[t][ct]));
                }
            }
        }
        __syncthreads();                                      // barrier 2
    }
    if (a.dS0 != nullptr) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int tc = wave + 4 * t;
            if (tc < NTC) {
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const f32x4 tr = quad_transpose4(accS[t][ct]);
                    *reinterpret_cast<f32x4*>(a.dS0 + (chain * DK + 16 * tc + 4 * grp + (l16 & 3)) * dv + j0 + 16 * ct + (l16 & ~3)) = tr;
                }
            }
        }
    }
}

bool gradmf_supported(int dk, int dv, bool bf16)
{
    return bf16 && (dk == 32 || dk == 64 || dk == 128) && (dv == 32 || dv == 64 || dv == 128);
}

template <int DK, int DV>
static void grad_launch(const GradVArgs& v, const GradKArgs& k, bool gbf16, dim3 grid, hipStream_t s)
{
    if (gbf16)
        hipLaunchKernelGGL((k_chunk_grad_mf<DK, DV, __bf16>), grid, dim3(kGvThreads), 0, s, v, k);
    else
        hipLaunchKernelGGL((k_chunk_grad_mf<DK, DV, float>), grid, dim3(kGvThreads), 0, s, v, k);
}

template <int DK>
static hipError_t grad_mf_dk(const GradVArgs& v, const GradKArgs& k, bool gbf16, hipStream_t s)
{
    const dim3 grid((unsigned)v.total);
    switch (v.dv) {
        case 32: grad_launch<DK, 32>(v, k, gbf16, grid, s); break;
        case 64: grad_launch<DK, 64>(v, k, gbf16, grid, s); break;
        case 128: grad_launch<DK, 128>(v, k, gbf16, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_chunk_state_bwd_mf(const BwdStateArgs& a, hipStream_t s)
{
    if (!gradmf_supported(a.dk, a.dv, true) || a.vs != 32 || a.nslices * 32 != a.dv || a.dSL != nullptr ||
        a.t_off == 0)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(a.B * a.H * a.nslices));
    switch (a.dk) {
        case 32: hipLaunchKernelGGL(k_chunk_state_bwd_mf<32>, grid, dim3(RsLds<32>::THREADS), 0, s, a); break;
        case 64: hipLaunchKernelGGL(k_chunk_state_bwd_mf<64>, grid, dim3(RsLds<64>::THREADS), 0, s, a); break;
        case 128: hipLaunchKernelGGL(k_chunk_state_bwd_mf<128>, grid, dim3(RsLds<128>::THREADS), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_chunk_grad_mf(const GradVArgs& v, const GradKArgs& k, bool gbf16, hipStream_t s)
{
    if (!gradmf_supported(v.dk, v.dv, true)) return hipErrorInvalidValue;
    switch (v.dk) {
        case 32: return grad_mf_dk<32>(v, k, gbf16, s);
        case 64: return grad_mf_dk<64>(v, k, gbf16, s);
        case 128: return grad_mf_dk<128>(v, k, gbf16, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn2
