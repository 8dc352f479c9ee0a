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

// Tg = gate dtype (alpha, b, w): float, or __bf16 with bf16 I/O
template <typename Tio, int DK, int VS, typename Tg>
__global__ __launch_bounds__(kThreads) void k_recurrent(RecArgs a)
{
    using IO = Io<Tio>;
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
                    x = g * IO::to_f(k[rowq + c]);
                }
                else if (which == 2) x = IO::to_f(k[rowq + c]);
                else x = IO::to_f(q[rowq + c]);
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
            u = w4 * ld_vec4(v + rowv);
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
            if (rg == 0) st_vec4(o + rowv, M + QK * delta);
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
    hipLaunchKernelGGL((k_recurrent<Tio, DK, VS, Tg>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
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
