// Output step of the GDN-2 layer on gfx950: the gated RMS norm that the
// burn-gdn2 0.1.9 README's "Architecture" diagram places after the core
// ("Gated RMS Norm <- SiLU Gate"), with norm_eps from its "Configuration":
//
//   y = o / sqrt(mean_j o_j^2 + eps) * weight_j * g_j * sigmoid(g_j)
//
// per (token, head) row of d_v channels, one weight vector for all heads.
//
// A row is handled by a group of P lanes (P = d_v / E rounded up to a power
// of two, at most a wave), E channels a lane in one 16-byte access (E = 8
// for bf16, 4 for fp32); every thread takes two rows whose loads are all
// issued first, so that four 16-byte loads a lane are in flight.  The sum of
// squares is reduced with shuffles inside the group, so every read of a row
// precedes its writes and y may alias o.  The kernel streams o, g and y
// once: HBM-bound.
#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"

namespace gdn2 {

template <typename Tio> struct Vec16;
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int E = 4; };
template <> struct Vec16<__bf16> { typedef bf16x8 type; static constexpr int E = 8; };

constexpr int kNormRowsPerThread = 2;

template <typename Tio, int P>
__global__ __launch_bounds__(kThreads) void k_gated_rmsnorm(NormArgs a)
{
    typedef typename Vec16<Tio>::type vec;
    constexpr int E = Vec16<Tio>::E;
    constexpr int R = kNormRowsPerThread;
    constexpr int RPB = kThreads / P * R;              // rows per workgroup
    const Tio* o = static_cast<const Tio*>(a.o);
    const Tio* g = static_cast<const Tio*>(a.g);
    Tio* y = static_cast<Tio*>(a.y);
    const int tid = threadIdx.x;
    const int c = E * (tid % P);
    const int cc = c < a.dv ? c : 0;
    // inactive lanes read a valid element and contribute nothing, so that
    // every lane of a group takes part in the shuffles
    int64_t off[R];
    bool act[R];
    vec ov[R], gv[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t row = (int64_t)blockIdx.x * RPB + i * (kThreads / P) + tid / P;
        act[i] = row < a.rows && c < a.dv;
        off[i] = (row < a.rows ? row : a.rows - 1) * a.dv + cc;
        ov[i] = *reinterpret_cast<const vec*>(o + off[i]);
        gv[i] = *reinterpret_cast<const vec*>(g + off[i]);
    }
    float wv[E];
#pragma unroll
    for (int e = 0; e < E; e += 4) {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(a.weight + cc + e);
        wv[e] = w4[0]; wv[e + 1] = w4[1]; wv[e + 2] = w4[2]; wv[e + 3] = w4[3];
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float x = (float)ov[i][e];
            ss += x * x;
        }
        if (!act[i]) ss = 0.f;
#pragma unroll
        for (int s = 1; s < P; s <<= 1) ss += __shfl_xor(ss, s, 64);
        const float r = __builtin_amdgcn_rsqf(ss * a.inv_dv + a.eps);
        if (act[i]) {
            vec out;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = (float)ov[i][e], z = (float)gv[i][e];
                out[e] = (Tio)(x * r * wv[e] * (z * sigmoid_f(z)));
            }
            *reinterpret_cast<vec*>(y + off[i]) = out;
        }
    }
}

template <typename Tio, int P>
static hipError_t norm_p(const NormArgs& a, hipStream_t s)
{
    constexpr int RPB = kThreads / P * kNormRowsPerThread;
    const int64_t nblk = (a.rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((k_gated_rmsnorm<Tio, P>), dim3((unsigned)nblk), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename Tio>
static hipError_t norm_t(const NormArgs& a, hipStream_t s)
{
    const int q = a.dv / Vec16<Tio>::E;                // dv is a multiple of 16
    if (q <= 2) return norm_p<Tio, 2>(a, s);
    if (q <= 4) return norm_p<Tio, 4>(a, s);
    if (q <= 8) return norm_p<Tio, 8>(a, s);
    if (q <= 16) return norm_p<Tio, 16>(a, s);
    if (q <= 32) return norm_p<Tio, 32>(a, s);
    return norm_p<Tio, 64>(a, s);
}

hipError_t launch_gated_rmsnorm(const NormArgs& a, bool bf16, hipStream_t s)
{
    return bf16 ? norm_t<__bf16>(a, s) : norm_t<float>(a, s);
}

}  // namespace gdn2
