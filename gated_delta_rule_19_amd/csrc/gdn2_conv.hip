// Short convolution of the GDN-2 layer's prologue on gfx950 (burn-gdn2 0.1.9
// README, "Architecture": a ShortConv on the projections before the L2 norm;
// "Configuration": use_short_conv, depthwise before the recurrence).  Causal
// and depthwise over tokens, K taps per channel, an optional SiLU, and K-1
// carried positions before the first token:
//
//   z[t, c] = sum_i w[c, i] xe[t - (K-1) + i, c],   y = z or z * sigmoid(z)
//
// Layout [B, T, C], channels fastest.  A lane takes 4 adjacent channels, so a
// wave reads 256 channels of one token row per access (1 KB fp32, 512 B
// bf16), and a tile of consecutive tokens together with the K-1 earlier
// positions it also needs; a tile issues all its loads before the
// arithmetic.  No contraction is large enough for the matrix cores (K <= 8
// taps a channel): both directions are HBM-bound, x and y (forward) or x, dy
// and dx (backward) crossing HBM once, the overlapping rows of neighbouring
// tiles mostly hitting in L2.
//
// Backward: a workgroup takes 256 channels of one 256-token span of one
// sequence; each wave walks 8 tiles of 8 tokens, recomputing z where the SiLU
// needs it, and writes dx (and, for the first tile of a sequence, the
// gradient of the carried state).  The weight gradient of a span is summed
// over its waves in LDS in a fixed order and written as one partial row; a
// second launch adds the rows in a fixed order, so dweight is reproducible.
#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"

namespace gdn2 {

constexpr int kConvCh = 4;                        // channels a lane
constexpr int kConvWaves = kThreads / 64;
constexpr int kConvTilesB = kConvSpan / (kConvWaves * kConvTileB);   // tiles a wave walks

static_assert(kConvTilesB * kConvWaves * kConvTileB == kConvSpan, "span must split into tiles");

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
    constexpr int TT = kConvTileF;
    constexpr int NR = TT + K - 1;
    const int64_t C4 = a.C / kConvCh;
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= a.B * a.ntile * C4) return;
    const int64_t c0 = (gid % C4) * kConvCh;
    const int64_t rest = gid / C4;
    const int64_t tile = rest % a.ntile, b = rest / a.ntile;
    const int64_t t0 = tile * TT, T = a.T, C = a.C;
    const Tio* x = static_cast<const Tio*>(a.x) + b * T * C + c0;
    const Tio* st = a.state_in ? static_cast<const Tio*>(a.state_in) + b * (K - 1) * C + c0 : nullptr;

    f32x4 r[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) r[j] = conv_row<Tio, K>(x, st, T, C, t0 - (K - 1) + j);
    // the carried window for a following call: only the first tile of a
    // sequence reads the state, so it alone writes the new one, after its reads
    const bool keep = K > 1 && a.state_out != nullptr && tile == 0;
    f32x4 so[K > 1 ? K - 1 : 1];
    if (keep) {
#pragma unroll
        for (int j = 0; j < K - 1; ++j) so[j] = conv_row<Tio, K>(x, st, T, C, T - (K - 1) + j);
    }
    f32x4 w[K];
    conv_taps<K>(a.weight, c0, w);

    Tio* y = static_cast<Tio*>(a.y) + b * T * C + c0;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        if (t0 + t < T) {
            f32x4 z = w[0] * r[t];
#pragma unroll
            for (int i = 1; i < K; ++i) z += w[i] * r[t + i];
            if (SILU) z = z * sigmoid4(z);
            st_vec4(y + (t0 + t) * C, z);
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
    constexpr int TT = kConvTileB;
    constexpr int NX = SILU ? TT + 2 * K - 2 : TT + K - 1;   // xe rows from t0 - (K-1)
    constexpr int ND = TT + K - 1;                           // dz rows from t0
    __shared__ f32x4 red[kConvWaves - 1][K][64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t C4 = a.C / kConvCh, ncb = (C4 + 63) / 64;
    int64_t blk = blockIdx.x;
    const int64_t cb = blk % ncb;
    blk /= ncb;
    const int64_t span = blk % a.nspan, b = blk / a.nspan;
    const int64_t c4 = cb * 64 + lane;
    const bool active = c4 < C4;
    const int64_t c0 = c4 * kConvCh, T = a.T, C = a.C;

    // acc[i]: weight gradient of tap i for the 4 channels
    f32x4 acc[K];
#pragma unroll
    for (int i = 0; i < K; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (active) {
        f32x4 w[K];
        conv_taps<K>(a.weight, c0, w);
        const Tio* x = static_cast<const Tio*>(a.x) + b * T * C + c0;
        const Tio* st = a.state_in ? static_cast<const Tio*>(a.state_in) + b * (K - 1) * C + c0 : nullptr;
        const Tio* dy = static_cast<const Tio*>(a.dy) + b * T * C + c0;
        Tio* dx = static_cast<Tio*>(a.dx) + b * T * C + c0;
#pragma unroll 1
        for (int n = 0; n < kConvTilesB; ++n) {
            const int64_t t0 = span * kConvSpan + (int64_t)(wave * kConvTilesB + n) * TT;
            const bool first = t0 == 0;   // also runs when T == 0, for the state's gradient
            if (t0 >= T && !first) break;
            f32x4 xr[NX], dz[ND];
#pragma unroll
            for (int j = 0; j < NX; ++j) xr[j] = conv_row<Tio, K>(x, st, T, C, t0 - (K - 1) + j);
#pragma unroll
            for (int j = 0; j < ND; ++j)
                dz[j] = (t0 + j < T) ? ld_vec4(dy + (t0 + j) * C) : f32x4{0.f, 0.f, 0.f, 0.f};
            if (SILU) {
                // d(z sigmoid z)/dz = s (1 + z (1 - s))
#pragma unroll
                for (int j = 0; j < ND; ++j) {
                    f32x4 z = w[0] * xr[j];
#pragma unroll
                    for (int i = 1; i < K; ++i) z += w[i] * xr[j + i];
                    const f32x4 s = sigmoid4(z);
                    dz[j] = dz[j] * s * (1.f + z * (1.f - s));
                }
            }
#pragma unroll
            for (int t = 0; t < TT; ++t) {
#pragma unroll
                for (int i = 0; i < K; ++i) acc[i] += dz[t] * xr[t + i];
            }
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                if (t0 + t < T) {
                    f32x4 g = w[K - 1] * dz[t];
#pragma unroll
                    for (int i = 0; i < K - 1; ++i) g += w[i] * dz[t + K - 1 - i];
                    st_vec4(dx + (t0 + t) * C, g);
                }
            }
            if (K > 1 && first && a.dstate != nullptr) {
                // positions q - (K-1) before the first token: taps i <= q reach dz[q - i]
                Tio* ds = static_cast<Tio*>(a.dstate) + b * (K - 1) * C + c0;
#pragma unroll
                for (int q = 0; q < K - 1; ++q) {
                    f32x4 g = w[q] * dz[0];
#pragma unroll
                    for (int i = 0; i < q; ++i) g += w[i] * dz[q - i];
                    st_vec4(ds + q * C, g);
                }
            }
        }
    }

    // the span's weight gradient: waves 1.. hand theirs to wave 0, which adds
    // them in wave order and writes one partial row [C][K]
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < K; ++i) red[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave == 0 && active) {
#pragma unroll
        for (int v = 0; v < kConvWaves - 1; ++v) {
#pragma unroll
            for (int i = 0; i < K; ++i) acc[i] += red[v][i][lane];
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

// dweight[e] = sum over the partial rows r = 0, 1, ... of part[r][e]
__global__ __launch_bounds__(kThreads) void k_conv_dw_sum(const float* part, float* dw, int64_t rows, int64_t n)
{
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e >= n) return;
    float s = 0.f;
    for (int64_t r = 0; r < rows; ++r) s += part[r * n + e];
    dw[e] = s;
}

namespace {

template <typename Tio, int K>
hipError_t conv_fwd_k(const ConvArgs& a, bool silu, hipStream_t s)
{
    const int64_t threads = a.B * a.ntile * (a.C / kConvCh);
    if (threads == 0) return hipSuccess;
    const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
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
    hipLaunchKernelGGL(k_conv_dw_sum, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                       a.part, a.dweight, a.B * a.nspan, n);
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
