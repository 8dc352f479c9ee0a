// Backward through the prologue options and shared query/key heads.
//
// The burn-gdn2 0.1.9 README ("Architecture") L2-normalises q and k before
// the mixer and activates the gates with a sigmoid; "Configuration" doubles
// b in negative-eigenvalue mode and lets several value heads share one
// query/key head (num_v_heads).  The core backward kernels take activated
// gates and one query/key row per value head, so for these options the
// library runs them on materialised inputs and maps the gradients back:
//
//   k_bwd_qk_pre    per query/key row x: xh = x / sqrt(|x|^2 + eps) (or x),
//                   written to each of the G value heads of its group;
//   k_gate_map<0>   gate logits z -> scale * sigmoid(z) as fp32
//                   (scale 2 for b in negative-eigenvalue mode, else 1);
//   k_bwd_qk_post   dxh = sum of the G value heads' gradients, then
//                   dx = (dxh - xh (xh . dxh)) / n with n = sqrt(|x|^2 + eps);
//   k_gate_map<1>   dz = dgate * scale * s (1 - s), s = sigmoid(z).
//
// Rows of dk channels are spread over dk/4 lanes (four channels each, one
// 16-byte or 8-byte access); the norms and dot products reduce across those
// lanes with xor shuffles.  The group sum runs in a fixed order, so the
// result is deterministic.
#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"

namespace gdn2 {

namespace {

constexpr int64_t kMaxGrid = 1 << 20;   // grid-stride loops beyond this many workgroups

// sum over the `lanes` consecutive lanes that hold one row (lanes a power of two <= 32)
__device__ __forceinline__ float row_sum(float x, int lanes)
{
    for (int off = 1; off < lanes; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

template <typename Tio>
__global__ void __launch_bounds__(kThreads) k_bwd_qk_pre(QkMapArgs a)
{
    const int lpr = a.dk / 4;                  // lanes per row
    const int rpw = kThreads / lpr;            // rows per workgroup
    const int sub = threadIdx.x % lpr;
    const bool l2 = a.l2;
    for (int64_t r = (int64_t)blockIdx.x * rpw + threadIdx.x / lpr; r - threadIdx.x / lpr < a.rows;
         r += (int64_t)gridDim.x * rpw) {
        const bool live = r < a.rows;
        const int64_t rr = live ? r : a.rows - 1;   // keep every lane in the shuffles
        const int64_t src = rr * a.dk + 4 * sub;
        f32x4 q = ld_vec4(static_cast<const Tio*>(a.q) + src);
        f32x4 k = ld_vec4(static_cast<const Tio*>(a.k) + src);
        if (l2) {
            const float sq = __builtin_amdgcn_rsqf(row_sum(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3],
                                                           lpr) + kL2normEps);
            const float sk = __builtin_amdgcn_rsqf(row_sum(k[0] * k[0] + k[1] * k[1] + k[2] * k[2] + k[3] * k[3],
                                                           lpr) + kL2normEps);
            q = q * sq;
            k = k * sk;
        }
        if (live) {
            for (int g = 0; g < a.G; ++g) {
                const int64_t dst = (rr * a.G + g) * a.dk + 4 * sub;
                st_vec4(static_cast<Tio*>(a.qh) + dst, q);
                st_vec4(static_cast<Tio*>(a.kh) + dst, k);
            }
        }
    }
}

template <typename Tio>
__global__ void __launch_bounds__(kThreads) k_bwd_qk_post(QkMapArgs a)
{
    const int lpr = a.dk / 4;
    const int rpw = kThreads / lpr;
    const int sub = threadIdx.x % lpr;
    const bool l2 = a.l2;
    for (int64_t r = (int64_t)blockIdx.x * rpw + threadIdx.x / lpr; r - threadIdx.x / lpr < a.rows;
         r += (int64_t)gridDim.x * rpw) {
        const bool live = r < a.rows;
        const int64_t rr = live ? r : a.rows - 1;
        const int64_t src = rr * a.dk + 4 * sub;
        f32x4 dq = {0.f, 0.f, 0.f, 0.f}, dk = dq;
        for (int g = 0; g < a.G; ++g) {
            const int64_t o = (rr * a.G + g) * a.dk + 4 * sub;
            dq += ld_vec4(static_cast<const Tio*>(a.dqh) + o);
            dk += ld_vec4(static_cast<const Tio*>(a.dkh) + o);
        }
        if (l2) {
            const f32x4 q = ld_vec4(static_cast<const Tio*>(a.q) + src);
            const f32x4 k = ld_vec4(static_cast<const Tio*>(a.k) + src);
            const float iq = __builtin_amdgcn_rsqf(row_sum(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3],
                                                           lpr) + kL2normEps);
            const float ik = __builtin_amdgcn_rsqf(row_sum(k[0] * k[0] + k[1] * k[1] + k[2] * k[2] + k[3] * k[3],
                                                           lpr) + kL2normEps);
            const f32x4 qh = q * iq, kh = k * ik;
            const float dotq = row_sum(qh[0] * dq[0] + qh[1] * dq[1] + qh[2] * dq[2] + qh[3] * dq[3], lpr);
            const float dotk = row_sum(kh[0] * dk[0] + kh[1] * dk[1] + kh[2] * dk[2] + kh[3] * dk[3], lpr);
            dq = (dq - qh * dotq) * iq;
            dk = (dk - kh * dotk) * ik;
        }
        if (live) {
            st_vec4(static_cast<Tio*>(a.dq) + src, dq);
            st_vec4(static_cast<Tio*>(a.dk_out) + src, dk);
        }
    }
}

__device__ __forceinline__ void st_gate4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void st_gate4(__bf16* p, f32x4 v)
{
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}

// POST = false: dst (fp32) = scale * sigmoid(z);  POST = true: dst (Tg) =
// grad (fp32) * scale * s (1 - s).  blockIdx.y picks one of the three gates.
template <typename Tg, bool POST>
__global__ void __launch_bounds__(kThreads) k_gate_map(GateMapArgs a)
{
    const int j = blockIdx.y;
    const Tg* z = static_cast<const Tg*>(a.z[j]);
    const float* gr = a.grad[j];
    const float scale = a.scale[j];
    const int64_t n4 = a.n[j] / 4;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads) {
        const f32x4 s = sigmoid4(ld_gate4(z + 4 * i));
        if (!POST) {
            st_gate4(static_cast<float*>(a.dst[j]) + 4 * i, s * scale);
        } else {
            const f32x4 d = *reinterpret_cast<const f32x4*>(gr + 4 * i);
            st_gate4(static_cast<Tg*>(a.dst[j]) + 4 * i, d * (s * (1.f - s)) * scale);
        }
    }
}

int64_t qk_grid(const QkMapArgs& a)
{
    const int64_t rpw = kThreads / (a.dk / 4);
    const int64_t g = (a.rows + rpw - 1) / rpw;
    return g < kMaxGrid ? g : kMaxGrid;
}

template <typename Tg>
hipError_t gate_launch(const GateMapArgs& a, bool post, hipStream_t s)
{
    int64_t n = a.n[0];
    for (int j = 1; j < 3; ++j) n = a.n[j] > n ? a.n[j] : n;
    if (n == 0) return hipSuccess;
    int64_t g = (n / 4 + kThreads - 1) / kThreads;
    g = g < kMaxGrid ? g : kMaxGrid;
    const dim3 grid((unsigned)g, 3);
    if (post) hipLaunchKernelGGL((k_gate_map<Tg, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_gate_map<Tg, false>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_qk_map(const QkMapArgs& a, bool post, bool bf16, hipStream_t s)
{
    if (a.rows == 0) return hipSuccess;
    const dim3 grid((unsigned)qk_grid(a)), block(kThreads);
    if (bf16) {
        if (post) hipLaunchKernelGGL(k_bwd_qk_post<__bf16>, grid, block, 0, s, a);
        else hipLaunchKernelGGL(k_bwd_qk_pre<__bf16>, grid, block, 0, s, a);
    } else {
        if (post) hipLaunchKernelGGL(k_bwd_qk_post<float>, grid, block, 0, s, a);
        else hipLaunchKernelGGL(k_bwd_qk_pre<float>, grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_gate_map(const GateMapArgs& a, bool post, bool gbf16, hipStream_t s)
{
    return gbf16 ? gate_launch<__bf16>(a, post, s) : gate_launch<float>(a, post, s);
}

}  // namespace gdn2
