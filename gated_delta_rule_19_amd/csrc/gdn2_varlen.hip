// Chunk plan of a packed variable-length batch on gfx950.
//
// The recurrence runs per sequence, each from its own state (burn-gdn2 0.1.9
// README, "Architecture" and "Quick start"), so the chunked form cuts every
// sequence into 64-token chunks that start at its first token.  One
// workgroup turns the caller's N+1 token offsets into the table the prep and
// state kernels index (layout in gdn2_launch.hpp):
//   cu[i]     offset i clamped into [0, T], then raised to the running
//             maximum, so lengths are never negative and sequences never
//             overlap whatever the caller passed;
//   first[i]  exclusive sum of ceil(length / 64): sequence i's first chunk;
//             first[N] is the chunk count, at most ceil(T/64) + N;
//   tab[c]    first token and length of chunk c.
// Offsets are scanned in tiles of one element per thread, carrying the
// running maximum and the running chunk sum from tile to tile.  Each chunk
// then finds its sequence by a binary search over first[] (the last
// sequence starting at or before it; an empty sequence shares its first
// chunk index with the next one, so the search lands on a non-empty one).
#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"

namespace gdn2 {

constexpr int kPlanThreads = 1024;
constexpr int kPlanLds = 4096;     // offsets and first chunks kept in LDS for the search

__global__ __launch_bounds__(kPlanThreads) void k_varlen_plan(PlanArgs a)
{
    __shared__ int sx[kPlanThreads];
    __shared__ int scu[kPlanLds], sfirst[kPlanLds];
    __shared__ int carry[2];
    const int tid = threadIdx.x;
    const int N = (int)a.N, T = (int)a.T;
    int* cu = a.plan;
    int* first = a.plan + (N + 1);
    int2* tab = reinterpret_cast<int2*>(a.plan + plan_head_words(N));
    auto clampT = [T](int x) { return x < 0 ? 0 : (x > T ? T : x); };

    if (tid == 0) carry[0] = carry[1] = 0;
    __syncthreads();
    for (int base = 0; base <= N; base += kPlanThreads) {
        const int i = base + tid;
        const int cmax = carry[0], csum = carry[1];
        // running maximum of the clamped offsets (lanes past N hold T; no
        // real lane's prefix includes them)
        int x = i <= N ? clampT(a.cu[i]) : T;
        sx[tid] = x;
        __syncthreads();
        for (int off = 1; off < kPlanThreads; off <<= 1) {
            const int y = tid >= off ? sx[tid - off] : x;
            __syncthreads();
            x = x > y ? x : y;
            sx[tid] = x;
            __syncthreads();
        }
        const int c = x > cmax ? x : cmax;
        int cn;                                         // clamped offset i + 1
        if (tid + 1 < kPlanThreads) {
            cn = sx[tid + 1] > cmax ? sx[tid + 1] : cmax;
        } else {
            const int nx = i + 1 <= N ? clampT(a.cu[i + 1]) : c;
            cn = nx > c ? nx : c;
        }
        const int nc = i < N ? (int)(((int64_t)cn - c + 63) / 64) : 0;
        __syncthreads();                                // sx is reused below
        // exclusive sum of the chunk counts
        int s = nc;
        sx[tid] = s;
        __syncthreads();
        for (int off = 1; off < kPlanThreads; off <<= 1) {
            const int y = tid >= off ? sx[tid - off] : 0;
            __syncthreads();
            s += y;
            sx[tid] = s;
            __syncthreads();
        }
        const int f = csum + s - nc;
        if (i <= N) {
            cu[i] = c;
            first[i] = f;
            if (i < kPlanLds) {
                scu[i] = c;
                sfirst[i] = f;
            }
        }
        __syncthreads();                                // every lane has read carry
        if (tid == kPlanThreads - 1) {
            carry[0] = c;
            carry[1] = f + nc;
        }
        __syncthreads();
    }

    // per-chunk token ranges (the table reads back what this workgroup wrote:
    // from LDS when it fits, else from global memory, ordered by the barrier)
    const int64_t total = carry[1];
    const int nchunks = (int)(total < a.ncmax ? total : a.ncmax);
    const bool lds = N + 1 <= kPlanLds;
    for (int gc = tid; gc < nchunks; gc += kPlanThreads) {
        int lo = 0, hi = N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            const int fm = lds ? sfirst[mid] : first[mid];
            if (fm <= gc) lo = mid;
            else hi = mid - 1;
        }
        const int f0 = lds ? sfirst[lo] : first[lo];
        const int c0 = lds ? scu[lo] : cu[lo], c1 = lds ? scu[lo + 1] : cu[lo + 1];
        const int t0 = c0 + 64 * (gc - f0);
        const int len = c1 - t0 < 64 ? c1 - t0 : 64;
        tab[gc] = make_int2(t0, len);
    }
}

hipError_t launch_varlen_plan(const PlanArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(k_varlen_plan, dim3(1), dim3(kPlanThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace gdn2
