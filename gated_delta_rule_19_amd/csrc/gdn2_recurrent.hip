// Fused recurrent forward / decode step of the GDN-2 token mixer on gfx950.
//
// Per token (burn-gdn2 0.1.9 README, "Architecture" recurrence):
//   S_t = (I - k (b*k)^T) diag(alpha) S + k (w*v)^T,   o_t = q^T S_t.
// Rewritten so that the state is read and written once per token:
//   X = diag(alpha) S
//   r = X^T (b*k),  m = X^T q            (two reductions over the key axis)
//   delta = w*v - r
//   S_t = X + k delta^T,  o_t = m + (q.k) delta
// since (I - k e^T) X = X - k (e^T X) and q^T k delta^T = (q.k) delta^T.
//
// Workgroup = (batch, head, value slice of VS columns), 256 threads.  Thread
// (jg, rg) holds columns 4*jg..4*jg+3 of rows rg, rg+NR, ... of the fp32
// state in registers for the whole call, so for a decode step (T = 1) the
// state streams from HBM and back exactly once with 16-byte accesses; a wave
// covers 64/NJ whole rows of the slice, contiguous in memory when VS == dv.
// The state is read and written with nontemporal (streaming) accesses: each
// byte is touched once per call, and keeping it out of the caches lets the
// write-back of one step overlap the reads of the next (about 14 % faster
// back to back on the B256 H16 d128 decode step).
// The key-axis vectors of token t+1 are fetched into LDS while token t is
// reduced; one barrier per token.
//
// Prologue flags: gate logits go through the sigmoid as they are fetched.
// With q/k L2 normalisation the reductions run on the raw q and k and also
// sum k^2 and q^2; r, m and q.k are then scaled by 1/|k|, 1/|q| and
// 1/(|q||k|) and the state update uses k/|k| -- the same values, with no
// extra pass over the key axis.
#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"

namespace gdn2 {

// Tg = gate dtype (alpha, b, w): float, or __bf16 with bf16 I/O; NT threads
// (256, or 512 for whole rows of 256 columns)
// CONV: the short convolution fused into the prologue (RecArgs conv_*):
// every thread keeps the last 3 raw inputs of the q/k channels it fetches
// and of its 4 value columns, and convolves each new token with them
template <typename Tio, int DK, int VS, typename Tg, int NT = kThreads, bool CONV = false>
__global__ __launch_bounds__(NT, NT == 512 ? 3 : 1) void k_recurrent(RecArgs a)
{
    using IO = Io<Tio>;
    constexpr int kThreads = NT;
    constexpr int NJ = VS / 4;                          // column groups (4 columns each)
    constexpr int NR = (kThreads / NJ) < DK ? (kThreads / NJ) : DK;   // row groups
    constexpr int NTH = NJ * NR;                        // threads holding state (multiple of 64)
    constexpr int RPT = DK / NR;                        // rows per thread
    constexpr int NW = NTH / 64;                        // waves holding state
    static_assert(NTH % 64 == 0 && NTH <= kThreads && DK % NR == 0, "thread layout");

    __shared__ __attribute__((aligned(16))) float vec[2][4][DK];   // alpha, b*k, k, q of a token
    __shared__ float red[2][NW][NJ][11];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const bool holder = tid < NTH;
    const int jg = tid % NJ, rg = tid / NJ;
    const int64_t chain = blockIdx.x / a.nslices;
    const int slice = (int)(blockIdx.x - chain * a.nslices);
    const int64_t bb = chain / a.H, hh = chain - bb * a.H;   // sequence, value head
    const int64_t hk = hh / (a.H / a.Hk);   // the query/key head this value head reads
    // the sequence's first packed token and its length (offsets of a packed
    // batch clamped into [0, T])
    int64_t tok0 = bb * a.T, tlen = a.T;
    if (a.cu != nullptr) {
        const int c0 = a.cu[bb], c1 = a.cu[bb + 1];
        tok0 = c0 < 0 ? 0 : (c0 > a.T ? a.T : c0);
        const int64_t e = c1 < tok0 ? tok0 : (c1 > a.T ? a.T : c1);
        tlen = e - tok0;
    }
    const int dv = a.dv;
    const int jc = slice * VS + 4 * jg;                 // first column of this thread
    const Tio* q = static_cast<const Tio*>(a.q);
    const Tio* k = static_cast<const Tio*>(a.k);
    const Tio* v = static_cast<const Tio*>(a.v);
    Tio* o = static_cast<Tio*>(a.o);
    const Tg* galpha = static_cast<const Tg*>(a.alpha);
    const Tg* gb = static_cast<const Tg*>(a.b);
    const Tg* gw = static_cast<const Tg*>(a.w);
    const bool logits = (a.flags & kFlagGateLogits) != 0;
    const bool l2norm = (a.flags & kFlagQkL2norm) != 0;
    const float bscale = (a.flags & kFlagNegEigval) ? 2.f : 1.f;

    f32x4 S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (holder && a.S_in != nullptr)
            S[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.S_in + (chain * DK + rg + NR * i) * dv + jc));
    }

    // key-axis vectors of a token -> registers (cooperative, coalesced)
    constexpr int VPT = (4 * DK + kThreads - 1) / kThreads;

    // fused convolution: taps right-aligned in 4 slots (zero below 4-K) and
    // the window of the 3 inputs before the next token (from conv_in before
    // the sequence), per fetched q/k element and per value column
    const int K = CONV ? a.conv_K : 1;
    const int64_t Hk = a.Hk;
    float kw[CONV ? VPT : 1][4], kh[CONV ? VPT : 1][3];
    f32x4 vw[4], vh[3];
    auto conv_tap = [&](int64_t c, int m) { return m >= 4 - K ? a.conv_w[c * K + m - (4 - K)] : 0.f; };
    auto conv_in = [&](int64_t c, int m) {   // input at position m - 3 < 0
        const int p = m - 3;
        if (p < -(K - 1) || a.conv_in == nullptr) return 0.f;
        return IO::to_f(static_cast<const Tio*>(a.conv_in)[(bb * (K - 1) + K - 1 + p) * a.conv_C + c]);
    };
    auto qk_chan = [&](int e) {   // conv channel of fetched element e (which 1, 2: k; 3: q)
        const int which = e / DK, c = e - which * DK;
        return which == 3 ? hk * DK + c : Hk * DK + hk * DK + c;
    };
    const int64_t vchan = 2 * Hk * DK + hh * a.dv + jc;
    if constexpr (CONV) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int e = tid + u * kThreads;
            if (e >= DK && e < 4 * DK) {
                const int64_t c = qk_chan(e);
#pragma unroll
                for (int m = 0; m < 4; ++m) kw[u][m] = conv_tap(c, m);
#pragma unroll
                for (int m = 0; m < 3; ++m) kh[u][m] = conv_in(c, m);
            }
        }
        if (holder) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) vw[m][e] = conv_tap(vchan + e, m);
#pragma unroll
            for (int m = 0; m < 3; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) vh[m][e] = conv_in(vchan + e, m);
        }
    }
    // one step of the window: the convolution at the new input x (fp32, SiLU
    // when asked, rounded to the I/O type as a stored convolution output)
    auto conv1 = [&](float (&h)[3], const float (&w)[4], float x) {
        float z = w[3] * x;
#pragma unroll
        for (int m = 0; m < 3; ++m) z += w[m] * h[m];
        h[0] = h[1];
        h[1] = h[2];
        h[2] = x;
        if (a.conv_silu) z *= sigmoid_f(z);
        return IO::to_f(IO::from_f(z));
    };

    auto fetch = [&](int64_t t, float (&st)[VPT]) {
        const int64_t rowk = ((tok0 + t) * a.H + hh) * DK;                    // gates: value head
        const int64_t rowq = ((tok0 + t) * a.Hk + hk) * DK;                   // q, k: its key head
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int e = tid + u * kThreads;
            float x = 0.f;
            if (e < 4 * DK) {
                const int which = e / DK, c = e - which * DK;
                if (which == 0) {
                    x = gate_f(galpha[rowk + c]);
                    if (logits) x = sigmoid_f(x);
                } else if (which == 1) {
                    float g = gate_f(gb[rowk + c]);
                    if (logits) g = sigmoid_f(g) * bscale;
                    if constexpr (CONV) x = g * conv1(kh[u], kw[u], IO::to_f(k[rowq + c]));
                    else x = g * IO::to_f(k[rowq + c]);
                }
                else if (which == 2) {
                    if constexpr (CONV) x = conv1(kh[u], kw[u], IO::to_f(k[rowq + c]));
                    else x = IO::to_f(k[rowq + c]);
                }
                else {
                    if constexpr (CONV) x = conv1(kh[u], kw[u], IO::to_f(q[rowq + c]));
                    else x = IO::to_f(q[rowq + c]);
                }
            }
            st[u] = x;
        }
    };
    auto stash = [&](int buf, const float (&st)[VPT]) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int e = tid + u * kThreads;
            if (e < 4 * DK) (&vec[buf][0][0])[e] = st[u];
        }
    };

    float stage[VPT];
    if (tlen > 0) {
        fetch(0, stage);
        stash(0, stage);
    }
    __syncthreads();

    for (int64_t t = 0; t < tlen; ++t) {
        const int buf = (int)(t & 1);
        if (t + 1 < tlen) fetch(t + 1, stage);
        const int64_t rowv = ((tok0 + t) * a.H + hh) * dv + jc;

        f32x4 u = {0.f, 0.f, 0.f, 0.f};
        f32x4 r = u, m = u;
        float qk = 0.f, k2 = 0.f, q2 = 0.f;
        float kreg[RPT];   // k of this thread's rows; vec[buf] is refilled for token t+2
                           // while slower waves may still be finishing token t
        if (holder) {
            f32x4 w4 = ld_gate4(gw + rowv);
            if (logits) w4 = sigmoid4(w4);
            if constexpr (CONV) {
                const f32x4 v4 = ld_vec4(v + rowv);
                f32x4 z = vw[3] * v4;
#pragma unroll
                for (int j = 0; j < 3; ++j) z += vw[j] * vh[j];
                vh[0] = vh[1];
                vh[1] = vh[2];
                vh[2] = v4;
                if (a.conv_silu) z = z * sigmoid4(z);
                u = w4 * IO::unpack4(IO::pack4(z));
            } else {
                u = w4 * ld_vec4(v + rowv);
            }
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int c = rg + NR * i;
                const float al = vec[buf][0][c], e = vec[buf][1][c];
                const float kk = vec[buf][2][c], qq = vec[buf][3][c];
                kreg[i] = kk;
                S[i] *= al;
                r += e * S[i];
                m += qq * S[i];
                qk += qq * kk;
                k2 += kk * kk;
                q2 += qq * qq;
            }
        }
        // reduce over the row groups of this wave (lanes sharing jg)
#pragma unroll
        for (int off = NJ; off < 64; off <<= 1) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                r[jj] += __shfl_xor(r[jj], off, 64);
                m[jj] += __shfl_xor(m[jj], off, 64);
            }
            qk += __shfl_xor(qk, off, 64);
            if (l2norm) {
                k2 += __shfl_xor(k2, off, 64);
                q2 += __shfl_xor(q2, off, 64);
            }
        }
        if (holder && lane < NJ) {
            float* dst = red[buf][wave][jg];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                dst[jj] = r[jj];
                dst[4 + jj] = m[jj];
            }
            dst[8] = qk;
            dst[9] = k2;
            dst[10] = q2;
        }
        if (t + 1 < tlen) stash(buf ^ 1, stage);
        __syncthreads();

        if (holder) {
            f32x4 R = {0.f, 0.f, 0.f, 0.f};
            f32x4 M = R;
            float QK = 0.f, K2 = 0.f, Q2 = 0.f;
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) {
                const float* src = red[buf][wv][jg];
                R += f32x4{src[0], src[1], src[2], src[3]};
                M += f32x4{src[4], src[5], src[6], src[7]};
                QK += src[8];
                K2 += src[9];
                Q2 += src[10];
            }
            float rk = 1.f;
            if (l2norm) {
                rk = __builtin_amdgcn_rsqf(K2 + kL2normEps);
                const float rq = __builtin_amdgcn_rsqf(Q2 + kL2normEps);
                R *= rk;
                M *= rq;
                QK *= rq * rk;
            }
            const f32x4 delta = u - R;
            const f32x4 ov = M + QK * delta;
            if (a.norm_g == nullptr) {
                if (rg == 0) st_vec4(o + rowv, ov);
            } else {
                // output step on the whole row (threads rg == 0, lanes 0..NJ-1 of
                // wave 0): sum of squares across the row, then the gated norm
                float ss = rg == 0 ? ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3] : 0.f;
#pragma unroll
                for (int off = 1; off < NJ; off <<= 1) ss += __shfl_xor(ss, off, 64);
                if (rg == 0) {
                    const float rn = __builtin_amdgcn_rsqf(ss * (1.f / (float)VS) + a.norm_eps);
                    const f32x4 z = ld_vec4(static_cast<const Tio*>(a.norm_g) + rowv);
                    const f32x4 wn = *reinterpret_cast<const f32x4*>(a.norm_w + jc);
                    f32x4 y;
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = ov[e] * rn * wn[e] * (z[e] * sigmoid_f(z[e]));
                    st_vec4(o + rowv, y);
                }
            }
            const f32x4 kd = rk * delta;
#pragma unroll
            for (int i = 0; i < RPT; ++i) S[i] += kreg[i] * kd;
        }
    }

    if (holder && a.S_out != nullptr) {
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            __builtin_nontemporal_store(S[i], reinterpret_cast<f32x4*>(a.S_out + (chain * DK + rg + NR * i) * dv + jc));
    }
    if constexpr (CONV) {
        // the window after the last token: the last K-1 inputs; q/k channels
        // by the first slice of the group's first value head, value columns
        // by row group 0 (conv_out does not overlap conv_in: other workgroups
        // may still be reading it)
        if (a.conv_out != nullptr && K > 1) {
            Tio* out = static_cast<Tio*>(a.conv_out) + bb * (K - 1) * a.conv_C;
            if (slice == 0 && hh % (a.H / a.Hk) == 0) {
#pragma unroll
                for (int u = 0; u < VPT; ++u) {
                    const int e = tid + u * kThreads;
                    if (e >= 2 * DK && e < 4 * DK) {   // the k and q elements
                        const int64_t c = qk_chan(e);
                        for (int j = 0; j < K - 1; ++j) out[j * a.conv_C + c] = IO::from_f(kh[u][3 - (K - 1) + j]);
                    }
                }
            }
            if (holder && rg == 0) {
                for (int j = 0; j < K - 1; ++j) {
                    const int m = 3 - (K - 1) + j;
                    st_vec4(out + j * a.conv_C + vchan, vh[m]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_decode: the same step for one token (T == 1, equal-length batches), built
// for streaming the state.  Every byte of the state is read once and written
// once, so the step is bound by how much state the CUs keep in flight and by
// how long each wave holds it without a request outstanding.  Each wave owns
// whole columns of the slice (all dk rows of VS / waves columns), so its
// reductions over the key axis stay inside the wave: no workgroup barrier,
// each wave reads the token's key-axis vectors into its own LDS rows.  Those
// vectors and w, v are requested before the state (so waiting for them never
// waits for the state), and k is read back from LDS for the update instead
// of being held per row, which keeps few registers beside the state.
// CONV: the short convolution fused into the prologue (RecArgs conv_*).  The
// workgroup convolves the token once: thread t takes channel t % dk of
// (alpha, k) or (b, q) and column t of the slice, requests their taps and
// window rows with the vectors (unconditionally: clamped addresses, values
// dropped by mask) and writes the results to one copy in LDS shared by the
// waves -- one workgroup barrier, after the state is requested.  The window
// after the token (the last K - 1 inputs) is written by the first slice of
// each key head's first value head (q/k channels) and by every slice (its
// columns).
// ---------------------------------------------------------------------------
template <typename Tio, int DK, int VS, typename Tg, int NT, int MINW, bool CONV = false>
__global__ __launch_bounds__(NT, MINW) void k_decode(RecArgs a)
{
    using IO = Io<Tio>;
    constexpr int NW = NT / 64;
    constexpr int WC = VS / NW;                         // columns per wave
    constexpr int NJ = WC / 4;                          // column groups of a wave
    constexpr int NR = 64 / NJ;                         // row groups of a wave
    constexpr int RPT = DK / NR;                        // rows per thread
    static_assert(VS % NW == 0 && WC % 4 == 0 && 64 % NJ == 0 && NR <= DK && DK % NR == 0, "thread layout");
    constexpr int VPL = 4 * DK / 64;                    // vector elements a lane loads

    __shared__ __attribute__((aligned(16))) float vec[CONV ? 1 : NW][4][DK];   // per wave (CONV: shared): alpha, b, k, q
    __shared__ __attribute__((aligned(16))) float vconv[CONV ? VS : 1];       // (CONV) the convolved values

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int jg = lane % NJ, rg = lane / NJ;
    const int64_t chain = blockIdx.x / a.nslices;
    const int slice = (int)(blockIdx.x - chain * a.nslices);
    const int64_t bb = chain / a.H, hh = chain - bb * a.H;
    const int64_t hk = hh / (a.H / a.Hk);
    const int dv = a.dv;
    const int jc = slice * VS + wave * WC + 4 * jg;
    const bool logits = (a.flags & kFlagGateLogits) != 0;
    const bool l2norm = (a.flags & kFlagQkL2norm) != 0;
    const float bscale = (a.flags & kFlagNegEigval) ? 2.f : 1.f;
    const Tg* galpha = static_cast<const Tg*>(a.alpha);
    const Tg* gb = static_cast<const Tg*>(a.b);
    const Tg* gw = static_cast<const Tg*>(a.w);
    const Tio* q = static_cast<const Tio*>(a.q);
    const Tio* k = static_cast<const Tio*>(a.k);
    float* vw = &vec[CONV ? 0 : wave][0][0];

    // 1. the token's key-axis vectors (this wave's copy) and the thread's w, v, before the state
    const int64_t rowk = (bb * a.H + hh) * DK, rowq = (bb * a.Hk + hk) * DK;
    float kv[CONV ? 1 : VPL];
#pragma unroll
    for (int u = 0; u < (CONV ? 0 : VPL); ++u) {
        const int e = lane + 64 * u;
        const int which = e / DK, c = e - which * DK;   // which is uniform per u when DK >= 64
        float x;
        if (which == 0) x = gate_f(galpha[rowk + c]);
        else if (which == 1) x = gate_f(gb[rowk + c]);
        else if (which == 2) x = IO::to_f(k[rowq + c]);
        else x = IO::to_f(q[rowq + c]);
        kv[u] = x;
    }
    const int64_t rowv = (bb * a.H + hh) * dv + jc;
    const auto wraw = *reinterpret_cast<const typename GateVec<Tg>::type*>(gw + rowv);
    const auto vraw = *reinterpret_cast<const typename IO::vec4*>(static_cast<const Tio*>(a.v) + rowv);
    // (CONV) thread t: channel c of pair P (0: alpha and k, 1: b and q) and
    // column ct of the slice; window row K-4+m holds the input at position
    // m - 3 (kept when that row exists and a window is given)
    const int K = CONV ? a.conv_K : 1;
    const Tio* cin = static_cast<const Tio*>(a.conv_in);
    const int t2 = tid < 2 * DK ? tid : 2 * DK - 1;
    const int P = __builtin_amdgcn_readfirstlane(t2 / DK), c = t2 - P * DK;   // P: wave-uniform (dk % 64 == 0)
    const int ct = tid < VS ? tid : VS - 1;
    const int64_t cch = P == 0 ? (a.Hk + hk) * DK + c : hk * DK + c;   // channel of k / q
    const int64_t vch = 2 * a.Hk * DK + hh * dv + slice * VS + ct;     // channel of the column
    float cg = 0.f, cx = 0.f, cv = 0.f, ctap[4], vtap[4], chis[3], vhis[3];
    bool keep[3];
    if constexpr (CONV) {
        static_assert(NT >= 2 * DK && NT >= VS, "one q/k element and one column per thread");
        cg = gate_f((P == 0 ? galpha : gb)[rowk + c]);
        cx = IO::to_f((P == 0 ? k : q)[rowq + c]);
        cv = IO::to_f(static_cast<const Tio*>(a.v)[(bb * a.H + hh) * dv + slice * VS + ct]);
        conv_taps1(a.conv_w, cch, K, ctap);
        conv_taps1(a.conv_w, vch, K, vtap);
        // dropped values are read from the weights (readable, and no value
        // the compiler already holds)
        const Tio* safe = reinterpret_cast<const Tio*>(a.conv_w);
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            keep[m] = K - 4 + m >= 0 && cin != nullptr;
            const int64_t wrow = (bb * (K - 1) + K - 4 + m) * a.conv_C;
            chis[m] = IO::to_f(*(keep[m] ? cin + wrow + cch : safe + cch));
            vhis[m] = IO::to_f(*(keep[m] ? cin + wrow + vch : safe + vch));
        }
    }
    // 2. the state
    f32x4 S[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.S_in != nullptr)
            S[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.S_in + (chain * DK + rg + NR * i) * dv + jc));
    }
    // 3. the vectors into this wave's LDS rows (read back by the same wave: no barrier)
    if constexpr (CONV) {
        // the convolution (fp32, SiLU when asked, rounded to the I/O type as
        // a stored convolution output would be) into the shared copy
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            chis[m] = keep_or_zero(chis[m], keep[m]);
            vhis[m] = keep_or_zero(vhis[m], keep[m]);
        }
        float zq = ctap[3] * cx, zv = vtap[3] * cv;
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            zq += ctap[m] * chis[m];
            zv += vtap[m] * vhis[m];
        }
        if (a.conv_silu) {
            zq *= sigmoid_f(zq);
            zv *= sigmoid_f(zv);
        }
        float g = cg;
        if (logits) g = P == 0 ? sigmoid_f(g) : sigmoid_f(g) * bscale;
        if (tid < 2 * DK) {
            vw[P * DK + c] = g;
            vw[(2 + P) * DK + c] = IO::to_f(IO::from_f(zq));
        }
        if (tid < VS) vconv[tid] = IO::to_f(IO::from_f(zv));
        __syncthreads();
    } else {
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
            const int e = lane + 64 * u;
            const int which = e / DK;
            float x = kv[u];
            if (logits && which == 0) x = sigmoid_f(x);
            if (logits && which == 1) x = sigmoid_f(x) * bscale;
            vw[e] = x;
        }
        __builtin_amdgcn_wave_barrier();
    }
    // 4. decay and the reductions over the key axis (row groups of the wave)
    f32x4 r = {0.f, 0.f, 0.f, 0.f}, m = r;
    float qk = 0.f, k2 = 0.f, q2 = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = rg + NR * i;
        const float al = vw[c], kk = vw[2 * DK + c], qq = vw[3 * DK + c];
        const float e = vw[DK + c] * kk;
        S[i] *= al;
        r += e * S[i];
        m += qq * S[i];
        qk += qq * kk;
        k2 += kk * kk;
        q2 += qq * qq;
    }
#pragma unroll
    for (int off = NJ; off < 64; off <<= 1) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            r[jj] += __shfl_xor(r[jj], off, 64);
            m[jj] += __shfl_xor(m[jj], off, 64);
        }
        qk += __shfl_xor(qk, off, 64);
        if (l2norm) {
            k2 += __shfl_xor(k2, off, 64);
            q2 += __shfl_xor(q2, off, 64);
        }
    }
    float rk = 1.f;
    if (l2norm) {
        rk = __builtin_amdgcn_rsqf(k2 + kL2normEps);
        const float rq = __builtin_amdgcn_rsqf(q2 + kL2normEps);
        r *= rk;
        m *= rq;
        qk *= rq * rk;
    }
    f32x4 w4 = widen4(wraw);
    if (logits) w4 = sigmoid4(w4);
    f32x4 v4;
    if constexpr (CONV) v4 = *reinterpret_cast<const f32x4*>(&vconv[wave * WC + 4 * jg]);
    else v4 = IO::unpack4(vraw);
    const f32x4 delta = w4 * v4 - r;
    // 5. the state update, streamed out
    const f32x4 kd = rk * delta;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        S[i] += vw[2 * DK + rg + NR * i] * kd;
        if (a.S_out != nullptr)
            __builtin_nontemporal_store(S[i], reinterpret_cast<f32x4*>(a.S_out + (chain * DK + rg + NR * i) * dv + jc));
    }
    // 6. the output row (optionally through the output step, whose row sum
    // spans the waves: one barrier, taken only then)
    const f32x4 ov = m + qk * delta;
    Tio* o = static_cast<Tio*>(a.o);
    if (a.norm_g == nullptr) {
        if (rg == 0) st_vec4(o + rowv, ov);
    } else {
        __shared__ float ssw[NW];
        float ss = rg == 0 ? ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3] : 0.f;
#pragma unroll
        for (int off = 1; off < NJ; off <<= 1) ss += __shfl_xor(ss, off, 64);
        if (lane == 0) ssw[wave] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) tot += ssw[wv];
        if (rg == 0) {
            const float rn = __builtin_amdgcn_rsqf(tot * (1.f / (float)VS) + a.norm_eps);
            const f32x4 z = ld_vec4(static_cast<const Tio*>(a.norm_g) + rowv);
            const f32x4 wn = *reinterpret_cast<const f32x4*>(a.norm_w + jc);
            f32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = ov[e] * rn * wn[e] * (z[e] * sigmoid_f(z[e]));
            st_vec4(o + rowv, y);
        }
    }
    if constexpr (CONV) {
        // 7. the window after the token: row j < K-1 holds the input at
        // position j - (K-2), slot 4-(K-1)+j of (h0, h1, h2, x)
        if (a.conv_out != nullptr && K > 1) {
            Tio* out = static_cast<Tio*>(a.conv_out) + bb * (K - 1) * a.conv_C;
            const bool qk = tid < 2 * DK && slice == 0 && hh % (a.H / a.Hk) == 0;
            for (int j = 0; j < K - 1; ++j) {
                const int sl = 4 - (K - 1) + j;   // 1..3
                if (qk) out[j * a.conv_C + cch] = IO::from_f(sl == 1 ? chis[1] : (sl == 2 ? chis[2] : cx));
                if (tid < VS) out[j * a.conv_C + vch] = IO::from_f(sl == 1 ? vhis[1] : (sl == 2 ? vhis[2] : cv));
            }
        }
    }
}

int recurrent_slice(int64_t nchains, int64_t T, int dv)
{
    // a decode step streams whole rows (widest slice); longer runs trade row
    // width for more independent workgroups
    static const int widths[4] = {128, 64, 32, 16};
    for (int i = 0; i < 4; ++i) {
        const int w = widths[i];
        if (dv % w) continue;
        if (T <= 1 || nchains * (dv / w) >= 1024 || w == 16) return w;
    }
    return 16;
}

template <typename Tio, int DK, int VS, typename Tg>
static hipError_t rec_v(const RecArgs& a, hipStream_t s)
{
    const int64_t nblk = a.B * a.H * (int64_t)a.nslices;
    if (a.conv_w != nullptr) {   // fused short convolution (equal-length batches)
        if (a.cu != nullptr || a.conv_K < 1 || a.conv_K > 4) return hipErrorInvalidValue;
        // the decode step: k_decode where its layout fits (dk >= 64)
        constexpr bool dec = DK >= 64 && (VS == 256 || (VS % 16 == 0 && VS >= 16 && (64 / (VS / 16)) <= DK));
        if constexpr (dec) {
            if (a.T == 1) {
                if constexpr (VS == 256)
                    hipLaunchKernelGGL((k_decode<Tio, DK, VS, Tg, 256, 2, true>), dim3((unsigned)nblk), dim3(256), 0, s, a);
                else
                    hipLaunchKernelGGL((k_decode<Tio, DK, VS, Tg, kThreads, (DK * VS >= 128 * 128 ? 4 : 8), true>),
                                       dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
                return hipGetLastError();
            }
        }
        if constexpr (VS == 256)
            hipLaunchKernelGGL((k_recurrent<Tio, DK, VS, Tg, 512, true>), dim3((unsigned)nblk), dim3(512), 0, s, a);
        else
            hipLaunchKernelGGL((k_recurrent<Tio, DK, VS, Tg, kThreads, true>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
        return hipGetLastError();
    }
    if constexpr (VS == 256) {
        // whole rows of 256 columns (the output step over dv = 256): 512 threads
        if (a.T == 1 && a.cu == nullptr)
            hipLaunchKernelGGL((k_decode<Tio, DK, VS, Tg, 256, 2>), dim3((unsigned)nblk), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_recurrent<Tio, DK, VS, Tg, 512>), dim3((unsigned)nblk), dim3(512), 0, s, a);
    } else {
        // every lane holds state rows: 64 / (columns per wave / 4) row groups at most dk
        constexpr bool fits = VS % 16 == 0 && VS >= 16 && (64 / (VS / 16)) <= DK && DK >= 64;
        if (fits && a.T == 1 && a.cu == nullptr) {
            if constexpr (fits)
                hipLaunchKernelGGL((k_decode<Tio, DK, VS, Tg, kThreads, (DK * VS >= 128 * 128 ? 4 : 8)>),
                                   dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
        } else {
            hipLaunchKernelGGL((k_recurrent<Tio, DK, VS, Tg>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
        }
    }
    return hipGetLastError();
}

template <typename Tio, int DK, typename Tg>
static hipError_t rec_dk(const RecArgs& a, int vs, hipStream_t s)
{
    switch (vs) {
        case 16: return rec_v<Tio, DK, 16, Tg>(a, s);
        case 32: return rec_v<Tio, DK, 32, Tg>(a, s);
        case 64: return rec_v<Tio, DK, 64, Tg>(a, s);
        case 128: return rec_v<Tio, DK, 128, Tg>(a, s);
        case 256: return rec_v<Tio, DK, 256, Tg>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename Tio, typename Tg>
static hipError_t rec_t(const RecArgs& a, int dk, int vs, hipStream_t s)
{
    switch (dk) {
        case 16: return rec_dk<Tio, 16, Tg>(a, vs, s);
        case 32: return rec_dk<Tio, 32, Tg>(a, vs, s);
        case 64: return rec_dk<Tio, 64, Tg>(a, vs, s);
        case 128: return rec_dk<Tio, 128, Tg>(a, vs, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_recurrent(const RecArgs& a, int dk, int vs, bool bf16, bool gbf16, hipStream_t s)
{
    if (!bf16) return gbf16 ? hipErrorInvalidValue : rec_t<float, float>(a, dk, vs, s);
    return gbf16 ? rec_t<__bf16, __bf16>(a, dk, vs, s) : rec_t<__bf16, float>(a, dk, vs, s);
}

}  // namespace gdn2
