// Short convolution of the GDN-2 layer's prologue on gfx950 (burn-gdn2 0.1.9
// README, "Architecture": a ShortConv on the projections before the L2 norm;
// "Configuration": use_short_conv, depthwise before the recurrence).  Causal
// and depthwise over tokens, K taps per channel, an optional SiLU, and K-1
// carried positions before the first token:
//
//   z[t, c] = sum_i w[c, i] xe[t - (K-1) + i, c],   y = z or z * sigmoid(z)
//
// Layout [B, T, C], channels fastest.  No contraction is large enough for the
// matrix cores (K <= 8 taps a channel): both directions are HBM-bound, x and
// y (forward) or x, dy and dx (backward) crossing HBM once.  A workgroup takes
// a block of 256 channels over a span of tokens: it first stages the span's
// rows (with the K-1 earlier positions, and for the backward the K-1 later
// ones) into LDS in 16-byte pieces, every load of the span issued before the
// first is used, so that a wave keeps many kilobytes in flight without
// holding them in registers; then each lane takes 4 channels of a quarter of
// the span from LDS.  A forward workgroup takes two consecutive spans, the
// second one's rows fetched into registers while the first is computed.
//
// Backward: a workgroup walks the sub-spans of a 128-token span, recomputing
// z where the SiLU needs it, writes dx (and, at the start of a sequence, the
// gradient of the carried state), and sums the span's weight gradient over
// its waves in LDS in a fixed order into one partial row; a second launch
// adds the rows in a fixed order, so dweight is reproducible.
#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"

namespace gdn2 {

constexpr int kConvCh = 4;                        // channels a lane
constexpr int kConvWaves = kThreads / 64;
constexpr int kConvBlk = 64 * kConvCh;            // channels a workgroup
constexpr int kConvSpansF = 2;                    // forward spans a workgroup

// rows of the channel block in LDS: 16-byte pieces of EPC elements
template <typename Tio> struct ConvRow {
    static constexpr int EPC = 16 / (int)sizeof(Tio);
    static constexpr int CHR = kConvBlk / EPC;    // pieces a row
};

// row of xe at token position p for the 4 channels at x / st: x past the end
// and a missing state read as zero
template <typename Tio, int K>
__device__ inline f32x4 conv_row(const Tio* x, const Tio* st, int64_t T, int64_t C, int64_t p)
{
    if (p >= 0) {
        if (p < T) return ld_vec4(x + p * C);
    } else if (st != nullptr) {
        return ld_vec4(st + (p + K - 1) * C);
    }
    return f32x4{0.f, 0.f, 0.f, 0.f};
}

// Stage NA rows of xe from position pa (x, the carried state before 0) and NB
// rows of a second tensor from position pb (zero outside [0, T)) for channels
// [c_lo, c_lo + 256) into LDS rows of 256 elements (zero past C).  Loads go
// out in batches of up to kConvBatch 16-byte pieces a thread, every load of a
// batch issued before its LDS writes.  x, st and y2 point at the sequence's
// base.
constexpr int kConvBatch = 10;

template <typename Tio, int K, int NA, int NB>
__device__ inline void conv_stage(Tio* lds, const Tio* x, const Tio* st, const Tio* y2, int64_t pa, int64_t pb,
                                  int64_t T, int64_t C, int64_t c_lo)
{
    constexpr int CHR = ConvRow<Tio>::CHR, EPC = ConvRow<Tio>::EPC;
    constexpr int N = (NA + NB) * CHR, PER = (N + kThreads - 1) / kThreads;
    constexpr int NB_ = (PER + kConvBatch - 1) / kConvBatch, BATCH = (PER + NB_ - 1) / NB_;
    typedef int __attribute__((ext_vector_type(4))) i32x4;
#pragma unroll
    for (int j0 = 0; j0 < PER; j0 += BATCH) {
        i32x4 v[BATCH];
#pragma unroll
        for (int jj = 0; jj < BATCH; ++jj) {
            const int id = threadIdx.x + (j0 + jj) * kThreads;
            v[jj] = i32x4{0, 0, 0, 0};
            const int row = id / CHR;
            const int64_t ch = c_lo + (int64_t)(id % CHR) * EPC;
            if (j0 + jj < PER && id < N && ch < C) {
                const Tio* src = nullptr;
                if (row < NA) {
                    const int64_t p = pa + row;
                    if (p >= 0) {
                        if (p < T) src = x + p * C + ch;
                    } else if (st != nullptr) {
                        src = st + (p + K - 1) * C + ch;
                    }
                } else {
                    const int64_t p = pb + (row - NA);
                    if (p >= 0 && p < T) src = y2 + p * C + ch;
                }
                if (src != nullptr) v[jj] = *reinterpret_cast<const i32x4*>(src);
            }
        }
#pragma unroll
        for (int jj = 0; jj < BATCH; ++jj) {
            const int id = threadIdx.x + (j0 + jj) * kThreads;
            if (j0 + jj < PER && id < N) reinterpret_cast<i32x4*>(lds)[id] = v[jj];
        }
        // keep the next batch's loads (and their registers) after these writes
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The same rows held in registers between a fetch and a put, so that the
// next sub-span's loads are in flight while the current one is computed.
template <typename Tio, int K, int NA, int NB>
struct ConvFetch {
    static constexpr int CHR = ConvRow<Tio>::CHR, EPC = ConvRow<Tio>::EPC;
    static constexpr int N = (NA + NB) * CHR, PER = (N + kThreads - 1) / kThreads;
    typedef int __attribute__((ext_vector_type(4))) i32x4;
    i32x4 v[PER];

    __device__ inline void fetch(const Tio* x, const Tio* st, const Tio* y2, int64_t pa, int64_t pb, int64_t T,
                                 int64_t C, int64_t c_lo)
    {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int id = threadIdx.x + j * kThreads;
            v[j] = i32x4{0, 0, 0, 0};
            const int row = id / CHR;
            const int64_t ch = c_lo + (int64_t)(id % CHR) * EPC;
            if (id < N && ch < C) {
                const Tio* src = nullptr;
                if (row < NA) {
                    const int64_t p = pa + row;
                    if (p >= 0) {
                        if (p < T) src = x + p * C + ch;
                    } else if (st != nullptr) {
                        src = st + (p + K - 1) * C + ch;
                    }
                } else {
                    const int64_t p = pb + (row - NA);
                    if (p >= 0 && p < T) src = y2 + p * C + ch;
                }
                if (src != nullptr) v[j] = *reinterpret_cast<const i32x4*>(src);
            }
        }
    }

    __device__ inline void put(Tio* lds) const
    {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int id = threadIdx.x + j * kThreads;
            if (id < N) reinterpret_cast<i32x4*>(lds)[id] = v[j];
        }
    }
};

// taps of the 4 channels from c0: w[i] holds tap i of each ([C][K] fp32 rows)
template <int K>
__device__ inline void conv_taps(const float* weight, int64_t c0, f32x4 (&w)[K])
{
    float f[kConvCh * K];
    const f32x4* src = reinterpret_cast<const f32x4*>(weight + c0 * K);
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const f32x4 v = src[j];
        f[4 * j] = v[0]; f[4 * j + 1] = v[1]; f[4 * j + 2] = v[2]; f[4 * j + 3] = v[3];
    }
#pragma unroll
    for (int i = 0; i < K; ++i) w[i] = f32x4{f[i], f[K + i], f[2 * K + i], f[3 * K + i]};
}

template <typename Tio, int K, bool SILU>
__global__ __launch_bounds__(kThreads) void k_short_conv(ConvArgs a)
{
    constexpr int S = kConvSpanF(sizeof(Tio) == 2);   // tokens a span
    constexpr int TW = S / kConvWaves;                 // tokens a wave
    constexpr int NR = S + K - 1;                      // staged rows from s0 - (K-1)
    __shared__ __align__(16) Tio lds[NR * kConvBlk];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t C4 = a.C / kConvCh, ncb = (C4 + 63) / 64;
    const int64_t ngrp = (a.ntile + kConvSpansF - 1) / kConvSpansF;
    int64_t blk = blockIdx.x;
    const int64_t cb = blk % ncb;
    blk /= ncb;
    const int64_t grp = blk % ngrp, b = blk / ngrp;
    const int64_t T = a.T, C = a.C;
    const int64_t c0 = (cb * 64 + lane) * kConvCh;
    const bool active = c0 < C;
    const Tio* x = static_cast<const Tio*>(a.x) + b * T * C;
    const Tio* st = a.state_in ? static_cast<const Tio*>(a.state_in) + b * (K - 1) * C : nullptr;
    Tio* y = static_cast<Tio*>(a.y) + b * T * C + c0;

    // the spans of a group go one after the other, the next one's rows
    // fetched into registers while the current one is computed
    ConvFetch<Tio, K, NR, 0> pf;
    pf.fetch(x, st, nullptr, grp * kConvSpansF * S - (K - 1), 0, T, C, cb * kConvBlk);
    // the carried window for a following call: only the first span of a
    // sequence reads the state, so its workgroup alone writes the new one,
    // after its reads
    const bool keep = K > 1 && a.state_out != nullptr && grp == 0 && wave == 0 && active;
    f32x4 so[K > 1 ? K - 1 : 1];
    if (keep) {
#pragma unroll
        for (int j = 0; j < K - 1; ++j)
            so[j] = conv_row<Tio, K>(x + c0, st ? st + c0 : nullptr, T, C, T - (K - 1) + j);
    }
    f32x4 w[K];
    if (active) conv_taps<K>(a.weight, c0, w);
    const Tio* row = lds + lane * kConvCh;
#pragma unroll 1
    for (int m = 0; m < kConvSpansF; ++m) {
        const int64_t span = grp * kConvSpansF + m;
        if (span >= a.ntile) break;         // uniform over the workgroup
        const int64_t s0 = span * S;
        if (m > 0) __syncthreads();         // the previous span's reads are done
        pf.put(lds);
        __syncthreads();
        if (m + 1 < kConvSpansF && span + 1 < a.ntile)
            pf.fetch(x, st, nullptr, s0 + S - (K - 1), 0, T, C, cb * kConvBlk);
        if (!active) continue;
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const int l = wave * TW + t;
            if (s0 + l < T) {
                f32x4 z = w[0] * ld_vec4(row + l * kConvBlk);
#pragma unroll
                for (int i = 1; i < K; ++i) z += w[i] * ld_vec4(row + (l + i) * kConvBlk);
                if (SILU) z = z * sigmoid4(z);
                st_vec4(y + (s0 + l) * C, z);
            }
        }
    }
    if (keep) {
        Tio* so_p = static_cast<Tio*>(a.state_out) + b * (K - 1) * C + c0;
#pragma unroll
        for (int j = 0; j < K - 1; ++j) st_vec4(so_p + j * C, so[j]);
    }
}

template <typename Tio, int K, bool SILU>
__global__ __launch_bounds__(kThreads) void k_short_conv_bwd(ConvBwdArgs a)
{
    constexpr int S = 32;                              // tokens a sub-span
    constexpr int NSUB = kConvSpan / S;
    constexpr int TW = S / kConvWaves;                 // tokens a wave
    constexpr int XR = SILU ? S + 2 * K - 2 : S + K - 1;   // staged xe rows from s0 - (K-1)
    constexpr int DR = S + K - 1;                          // staged dy rows from s0
    // with the SiLU, dz = dy * d(z sigmoid z)/dz is formed once a row: in place
    // of dy for fp32, in an fp32 area for bf16
    constexpr bool SEP = SILU && sizeof(Tio) == 2;
    constexpr int LDS_IO = (XR + DR) * kConvBlk * (int)sizeof(Tio);
    constexpr int LDS_RED = (kConvWaves - 1) * K * 64 * 16;
    constexpr int LDS_A = LDS_IO > LDS_RED ? LDS_IO : LDS_RED;
    static_assert(NSUB * S == kConvSpan, "span must split into sub-spans");
    __shared__ __align__(16) char lds_a[LDS_A];
    __shared__ __align__(16) f32x4 dzs[SEP ? DR * 64 : 1];
    Tio* lds = reinterpret_cast<Tio*>(lds_a);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t C4 = a.C / kConvCh, ncb = (C4 + 63) / 64;
    int64_t blk = blockIdx.x;
    const int64_t cb = blk % ncb;
    blk /= ncb;
    const int64_t span = blk % a.nspan, b = blk / a.nspan;
    const int64_t T = a.T, C = a.C;
    const int64_t c0 = (cb * 64 + lane) * kConvCh;
    const bool active = c0 < C;
    const Tio* x = static_cast<const Tio*>(a.x) + b * T * C;
    const Tio* st = a.state_in ? static_cast<const Tio*>(a.state_in) + b * (K - 1) * C : nullptr;
    const Tio* dy = static_cast<const Tio*>(a.dy) + b * T * C;
    Tio* dx = static_cast<Tio*>(a.dx) + b * T * C + c0;

    f32x4 w[K], acc[K];   // acc[i]: weight gradient of tap i for the 4 channels
#pragma unroll
    for (int i = 0; i < K; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (active) conv_taps<K>(a.weight, c0, w);

    Tio* xrow = lds + lane * kConvCh;
    Tio* drow = lds + XR * kConvBlk + lane * kConvCh;
    // dz of staged row j (row j = position s0 + j)
    auto dz_at = [&](int j) -> f32x4 {
        if constexpr (SEP) return dzs[j * 64 + lane];
        else return ld_vec4(drow + j * kConvBlk);
    };
    // bf16 rows are few enough a thread to be prefetched in registers
    constexpr bool PIPE = sizeof(Tio) == 2;
    ConvFetch<Tio, K, XR, DR> pf;
    if constexpr (PIPE) pf.fetch(x, st, dy, span * kConvSpan - (K - 1), span * kConvSpan, T, C, cb * kConvBlk);
#pragma unroll 1
    for (int n = 0; n < NSUB; ++n) {
        const int64_t s0 = span * kConvSpan + (int64_t)n * S;
        if (s0 >= T && s0 != 0) break;      // uniform over the workgroup; T == 0 still runs once
        if (n > 0) __syncthreads();         // the previous sub-span's reads are done
        if constexpr (PIPE) {
            pf.put(lds);
            __syncthreads();
            const int64_t s1 = s0 + S;
            if (n + 1 < NSUB && s1 < T) pf.fetch(x, st, dy, s1 - (K - 1), s1, T, C, cb * kConvBlk);
        } else {
            conv_stage<Tio, K, XR, DR>(lds, x, st, dy, s0 - (K - 1), s0, T, C, cb * kConvBlk);
            __syncthreads();
        }
        if (SILU) {
            // rows past T hold dy = 0, so their dz is 0
            if (active) {
#pragma unroll
                for (int j = wave; j < DR; j += kConvWaves) {
                    f32x4 z = w[0] * ld_vec4(xrow + j * kConvBlk);
#pragma unroll
                    for (int i = 1; i < K; ++i) z += w[i] * ld_vec4(xrow + (j + i) * kConvBlk);
                    const f32x4 sg = sigmoid4(z);
                    const f32x4 d = ld_vec4(drow + j * kConvBlk) * sg * (1.f + z * (1.f - sg));
                    if constexpr (SEP) dzs[j * 64 + lane] = d;
                    else st_vec4(drow + j * kConvBlk, d);
                }
            }
            __syncthreads();
        }
        if (!active) continue;
        const int l0 = wave * TW;
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const f32x4 d = dz_at(l0 + t);
#pragma unroll
            for (int i = 0; i < K; ++i) acc[i] += d * ld_vec4(xrow + (l0 + t + i) * kConvBlk);
        }
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const int64_t p = s0 + l0 + t;
            if (p < T) {
                f32x4 g = w[K - 1] * dz_at(l0 + t);
#pragma unroll
                for (int i = 0; i < K - 1; ++i) g += w[i] * dz_at(l0 + t + K - 1 - i);
                // the window after the last token holds positions T-(K-1)..T-1
                if (K > 1 && a.dstate_out != nullptr && p >= T - (K - 1))
                    g += ld_vec4(static_cast<const Tio*>(a.dstate_out) + (b * (K - 1) + p - T + K - 1) * C + c0);
                st_vec4(dx + p * C, g);
            }
        }
        if (K > 1 && s0 + l0 == 0 && a.dstate != nullptr) {
            // positions q - (K-1) before the first token: taps i <= q reach dz[q - i]
            Tio* ds = static_cast<Tio*>(a.dstate) + b * (K - 1) * C + c0;
#pragma unroll
            for (int q = 0; q < K - 1; ++q) {
                f32x4 g = w[q] * dz_at(0);
#pragma unroll
                for (int i = 0; i < q; ++i) g += w[i] * dz_at(q - i);
                // with T < K-1 the window after the last token still holds
                // state inputs: position q-(K-1) is its row q - T
                if (a.dstate_out != nullptr && q >= T)
                    g += ld_vec4(static_cast<const Tio*>(a.dstate_out) + (b * (K - 1) + q - T) * C + c0);
                st_vec4(ds + q * C, g);
            }
        }
    }

    // the span's weight gradient: waves 1.. hand theirs to wave 0 (in the
    // staging area, once every wave is done with it), which adds them in wave
    // order and writes one partial row [C][K]
    f32x4* red = reinterpret_cast<f32x4*>(lds_a);   // [wave - 1][K][64]
    __syncthreads();
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < K; ++i) red[((wave - 1) * K + i) * 64 + lane] = acc[i];
    }
    __syncthreads();
    if (wave == 0 && active) {
#pragma unroll
        for (int v = 0; v < kConvWaves - 1; ++v) {
#pragma unroll
            for (int i = 0; i < K; ++i) acc[i] += red[(v * K + i) * 64 + lane];
        }
        float f[kConvCh * K];
#pragma unroll
        for (int j = 0; j < kConvCh; ++j) {
#pragma unroll
            for (int i = 0; i < K; ++i) f[j * K + i] = acc[i][j];
        }
        f32x4* dst = reinterpret_cast<f32x4*>(a.part + (b * a.nspan + span) * C * K + c0 * K);
#pragma unroll
        for (int j = 0; j < K; ++j) dst[j] = f32x4{f[4 * j], f[4 * j + 1], f[4 * j + 2], f[4 * j + 3]};
    }
}

// dweight[e] = sum over the partial rows r = 0, 1, ... of part[r][e], added
// in row order; 16 rows' loads are in flight at a time
constexpr int kConvSumThreads = 64;

__global__ __launch_bounds__(kConvSumThreads) void k_conv_dw_sum(const float* part, float* dw, int64_t rows,
                                                                 int64_t n)
{
    const int64_t e = (int64_t)blockIdx.x * kConvSumThreads + threadIdx.x;
    if (e >= n) return;
    float s = 0.f;
    int64_t r = 0;
    for (; r + 16 <= rows; r += 16) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = part[(r + j) * n + e];
#pragma unroll
        for (int j = 0; j < 16; ++j) s += v[j];
    }
    for (; r < rows; ++r) s += part[r * n + e];
    dw[e] = s;
}

namespace {

template <typename Tio, int K>
hipError_t conv_fwd_k(const ConvArgs& a, bool silu, hipStream_t s)
{
    const int64_t blocks = a.B * ((a.ntile + kConvSpansF - 1) / kConvSpansF) * ((a.C / kConvCh + 63) / 64);
    if (blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks);
    if (silu)
        hipLaunchKernelGGL((k_short_conv<Tio, K, true>), grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((k_short_conv<Tio, K, false>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename Tio, int K>
hipError_t conv_bwd_k(const ConvBwdArgs& a, bool silu, hipStream_t s)
{
    const int64_t ncb = (a.C / kConvCh + 63) / 64;
    const int64_t blocks = a.B * a.nspan * ncb;
    if (blocks > 0) {
        if (silu)
            hipLaunchKernelGGL((k_short_conv_bwd<Tio, K, true>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((k_short_conv_bwd<Tio, K, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t n = a.C * K;
    hipLaunchKernelGGL(k_conv_dw_sum, dim3((unsigned)((n + kConvSumThreads - 1) / kConvSumThreads)),
                       dim3(kConvSumThreads), 0, s, a.part, a.dweight, a.B * a.nspan, n);
    return hipGetLastError();
}

template <typename Tio>
hipError_t conv_fwd_t(const ConvArgs& a, int K, bool silu, hipStream_t s)
{
    switch (K) {
        case 1: return conv_fwd_k<Tio, 1>(a, silu, s);
        case 2: return conv_fwd_k<Tio, 2>(a, silu, s);
        case 3: return conv_fwd_k<Tio, 3>(a, silu, s);
        case 4: return conv_fwd_k<Tio, 4>(a, silu, s);
        case 5: return conv_fwd_k<Tio, 5>(a, silu, s);
        case 6: return conv_fwd_k<Tio, 6>(a, silu, s);
        case 7: return conv_fwd_k<Tio, 7>(a, silu, s);
        case 8: return conv_fwd_k<Tio, 8>(a, silu, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename Tio>
hipError_t conv_bwd_t(const ConvBwdArgs& a, int K, bool silu, hipStream_t s)
{
    switch (K) {
        case 1: return conv_bwd_k<Tio, 1>(a, silu, s);
        case 2: return conv_bwd_k<Tio, 2>(a, silu, s);
        case 3: return conv_bwd_k<Tio, 3>(a, silu, s);
        case 4: return conv_bwd_k<Tio, 4>(a, silu, s);
        case 5: return conv_bwd_k<Tio, 5>(a, silu, s);
        case 6: return conv_bwd_k<Tio, 6>(a, silu, s);
        case 7: return conv_bwd_k<Tio, 7>(a, silu, s);
        case 8: return conv_bwd_k<Tio, 8>(a, silu, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_short_conv(const ConvArgs& a, int K, bool silu, bool bf16, hipStream_t s)
{
    return bf16 ? conv_fwd_t<__bf16>(a, K, silu, s) : conv_fwd_t<float>(a, K, silu, s);
}

hipError_t launch_short_conv_bwd(const ConvBwdArgs& a, int K, bool silu, bool bf16, hipStream_t s)
{
    return bf16 ? conv_bwd_t<__bf16>(a, K, silu, s) : conv_bwd_t<float>(a, K, silu, s);
}

}  // namespace gdn2
