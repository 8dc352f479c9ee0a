// Device helpers shared by the GDN-2 kernels (gfx950 / CDNA4, wave64).
//
// Matrix-core convention used everywhere in this library.  A 16x16 output
// tile D = A (16 x K) * B (K x 16) is accumulated by "K-blocks".  In every
// K-block each lane supplies 16 bytes of A and 16 bytes of B:
//   A: row  m = lane % 16, elements k0 + EPL*(lane/16) .. +EPL-1 of that row
//   B: col  n = lane % 16, elements k0 + EPL*(lane/16) .. +EPL-1 of that column
// where EPL = 8 for bf16 (one v_mfma_f32_16x16x32_bf16, K-block = 32) and
// EPL = 4 for fp32 (four v_mfma_f32_16x16x4_f32, K-block = 16; the i-th
// instruction takes element i of every lane).  Because A and B use the same
// lane->k assignment, the sum runs over every k of the block exactly once.
// The accumulator holds D[4*(lane/16) + i][lane % 16], i = 0..3.
//
// So an operand stored with its K index contiguous (row-major A, or B stored
// as B^T) is fetched with one 16-byte load per lane per K-block, from LDS or
// global memory alike.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

constexpr int kThreads = 256;   // every kernel runs 4 waves of 64 lanes
constexpr int kChunk = 64;      // chunk length of the chunked form

__host__ __device__ constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }

// ---------------------------------------------------------------------------
// Element type traits: Tio is float (fp32 I/O) or __bf16 (bf16 I/O).
// ---------------------------------------------------------------------------
template <typename T> struct Io;

template <> struct Io<float> {
    static constexpr int EPL = 4;        // elements per lane per K-block
    static constexpr int KB = 16;        // K per K-block
    typedef f32x4 frag;                  // 16 bytes
    typedef f32x4 vec4;                  // 4 elements
    typedef f32x2 pair;                  // 2 elements
    __device__ static inline float to_f(float x) { return x; }
    __device__ static inline f32x2 pair_f(pair p) { return p; }
    __device__ static inline pair pack2(float x, float y) { return f32x2{x, y}; }
    __device__ static inline float from_f(float x) { return x; }
    __device__ static inline vec4 pack4(f32x4 v) { return v; }
    __device__ static inline f32x4 unpack4(vec4 v) { return v; }
    __device__ static inline f32x4 mma(f32x4 acc, frag a, frag b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
        return acc;
    }
    // multiply the EPL elements of a fragment by per-k factors f[0..EPL-1]
    __device__ static inline frag scale(frag a, const float* f) {
        f32x4 s = *reinterpret_cast<const f32x4*>(f);
        return a * s;
    }
};

template <> struct Io<__bf16> {
    static constexpr int EPL = 8;
    static constexpr int KB = 32;
    typedef bf16x8 frag;
    typedef bf16x4 vec4;
    typedef bf16x2 pair;
    __device__ static inline float to_f(__bf16 x) { return (float)x; }
    __device__ static inline f32x2 pair_f(pair p) { return f32x2{(float)p[0], (float)p[1]}; }
    __device__ static inline pair pack2(float x, float y) {
        pair r;
        r[0] = (__bf16)x; r[1] = (__bf16)y;
        return r;
    }
    __device__ static inline __bf16 from_f(float x) { return (__bf16)x; }   // RNE (v_cvt_pk_bf16_f32)
    __device__ static inline vec4 pack4(f32x4 v) {
        vec4 r;
        r[0] = (__bf16)v[0]; r[1] = (__bf16)v[1]; r[2] = (__bf16)v[2]; r[3] = (__bf16)v[3];
        return r;
    }
    __device__ static inline f32x4 unpack4(vec4 v) {
        f32x4 r = {(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
        return r;
    }
    __device__ static inline f32x4 mma(f32x4 acc, frag a, frag b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    __device__ static inline frag scale(frag a, const float* f) {
        f32x4 s0 = *reinterpret_cast<const f32x4*>(f);
        f32x4 s1 = *reinterpret_cast<const f32x4*>(f + 4);
        frag r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r[i] = (__bf16)((float)a[i] * s0[i]);
            r[4 + i] = (__bf16)((float)a[4 + i] * s1[i]);
        }
        return r;
    }
};

template <typename T>
__device__ inline typename Io<T>::frag ld_frag(const T* p) {
    return *reinterpret_cast<const typename Io<T>::frag*>(p);
}

template <typename T>
__device__ inline void st_vec4(T* p, f32x4 v) {
    *reinterpret_cast<typename Io<T>::vec4*>(p) = Io<T>::pack4(v);
}

template <typename T>
__device__ inline f32x4 ld_vec4(const T* p) {
    return Io<T>::unpack4(*reinterpret_cast<const typename Io<T>::vec4*>(p));
}

__device__ inline float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Within every group of four consecutive lanes, transpose the 4 x 4 matrix
// whose rows are the lanes and whose columns are the registers: lane q gets
// register q of the four lanes, in lane order.  Two rounds of register swaps
// between lane pairs (lane ^ 2, then lane ^ 1) through DPP quad permutations;
// every lane of the wave must be active.
__device__ inline f32x4 quad_transpose4(f32x4 v)
{
    const int q = threadIdx.x & 3;
    const auto swap2 = [](float x) {     // quad_perm [2, 3, 0, 1]
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
    };
    const auto swap1 = [](float x) {     // quad_perm [1, 0, 3, 2]
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
    };
    // lanes q, q ^ 2 exchange the registers whose bit 1 differs from q's
    const bool hi = (q & 2) != 0;
    float s0 = swap2(hi ? v[0] : v[2]), s1 = swap2(hi ? v[1] : v[3]);
    if (hi) { v[0] = s0; v[1] = s1; } else { v[2] = s0; v[3] = s1; }
    // lanes q, q ^ 1 exchange the registers whose bit 0 differs from q's
    const bool odd = (q & 1) != 0;
    s0 = swap1(odd ? v[0] : v[1]);
    s1 = swap1(odd ? v[2] : v[3]);
    if (odd) { v[0] = s0; v[2] = s1; } else { v[1] = s0; v[3] = s1; }
    return v;
}

// ---------------------------------------------------------------------------
// Gates: fp32 or bf16 in memory, fp32 in registers.  Prologue flags
// (GDN2_FLAG_* of gdn2.h) are passed to the kernels as plain ints.
// ---------------------------------------------------------------------------
constexpr int kFlagGateLogits = 1, kFlagNegEigval = 2, kFlagQkL2norm = 4;
constexpr float kL2normEps = 1e-6f;
// Smallest decay the chunked mode uses: alpha below it (zero included) is
// raised to it, so that a product of 4 consecutive decays stays >= 2^-80 and
// its inverse stays finite in fp32 and bf16.  A raised alpha keeps at most a
// 2^-20 share of the state it should have erased.
constexpr float kAlphaFloor = 0x1p-20f;
__device__ inline f32x4 alpha_floor4(f32x4 a)
{
    return f32x4{fmaxf(a[0], kAlphaFloor), fmaxf(a[1], kAlphaFloor), fmaxf(a[2], kAlphaFloor),
                 fmaxf(a[3], kAlphaFloor)};
}

__device__ inline float gate_f(float x) { return x; }
__device__ inline float gate_f(__bf16 x) { return (float)x; }

template <typename Tg> struct GateVec;
template <> struct GateVec<float> { typedef f32x4 type; };
template <> struct GateVec<__bf16> { typedef bf16x4 type; };

// four consecutive gates, widened to fp32
__device__ inline f32x4 ld_gate4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ inline f32x4 ld_gate4(const __bf16* p)
{
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

__device__ inline f32x4 widen4(f32x4 v) { return v; }
__device__ inline f32x4 widen4(bf16x4 v) { return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]}; }

// logistic function 1 / (1 + exp(-x)); saturates to 0 / 1 for large |x|
__device__ inline float sigmoid_f(float x) { return fast_rcp(1.f + __expf(-x)); }
__device__ inline f32x4 sigmoid4(f32x4 x)
{
    return f32x4{sigmoid_f(x[0]), sigmoid_f(x[1]), sigmoid_f(x[2]), sigmoid_f(x[3])};
}

// ---- short convolution taps (weight [C][K] fp32, 1 <= K <= 4) -------------
// Taps are right-aligned in 4 slots, w[m] = weight[c][m - (4 - K)] for
// m >= 4 - K and 0 below, so that z[t] = sum_m w[m] x[t - 3 + m] for any K.
// Every load is unconditional (indices clamped into the row) and the slots
// are chosen afterwards with bit masks: a load under a branch, or a value
// picked by one, would drain the vector-memory counter together with every
// other load in flight.
// The 4K weights of 4 consecutive channels c..c+3 (c % 4 == 0) are contiguous
// and 16-byte aligned: K vector loads, then conv_taps4_pick.
__device__ inline void conv_taps4_load(const float* weight, int64_t c, int K, f32x4 (&f)[4])
{
    const f32x4* src = reinterpret_cast<const f32x4*>(weight + c * K);
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = src[j < K ? j : K - 1];
}
__device__ inline void conv_taps4_pick(int K, const f32x4 (&f)[4], f32x4 (&w)[4])
{
    const unsigned m4 = 0u - (unsigned)(K == 4), m3 = 0u - (unsigned)(K == 3);
    const unsigned m2 = 0u - (unsigned)(K == 2), m1 = 0u - (unsigned)(K == 1);
    auto at = [&](int i) { return __float_as_uint(f[i / 4][i % 4]); };   // weight[c + i / K][i % K]
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            unsigned u = at(4 * e + m) & m4;
            if (m >= 1) u |= at(3 * e + m - 1) & m3;
            if (m >= 2) u |= at(2 * e + m - 2) & m2;
            if (m == 3) u |= at(e) & m1;
            w[m][e] = __uint_as_float(u);
        }
}
// the taps of one channel c
__device__ inline void conv_taps1(const float* weight, int64_t c, int K, float (&w)[4])
{
    float f[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = weight[c * K + (j < K ? j : K - 1)];
    const unsigned m4 = 0u - (unsigned)(K == 4), m3 = 0u - (unsigned)(K == 3);
    const unsigned m2 = 0u - (unsigned)(K == 2), m1 = 0u - (unsigned)(K == 1);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        unsigned u = __float_as_uint(f[m]) & m4;
        if (m >= 1) u |= __float_as_uint(f[m - 1]) & m3;
        if (m >= 2) u |= __float_as_uint(f[m - 2]) & m2;
        if (m == 3) u |= __float_as_uint(f[0]) & m1;
        w[m] = __uint_as_float(u);
    }
}
// x where keep holds, else all-zero bits (no branch)
template <typename V>
__device__ inline V keep_or_zero(V x, bool keep)
{
    static_assert(sizeof(V) % 4 == 0, "whole 32-bit words");
    const unsigned mk = 0u - (unsigned)keep;
    V r;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(V) / 4); ++i)
        reinterpret_cast<unsigned*>(&r)[i] = reinterpret_cast<const unsigned*>(&x)[i] & mk;
    return r;
}
__device__ inline float keep_or_zero(float x, bool keep)
{
    return __uint_as_float(__float_as_uint(x) & (0u - (unsigned)keep));
}

// ---------------------------------------------------------------------------
// Where chunks lie in the token tensors and the workspace.  Equal-length
// batches (plan == nullptr): chain (sequence bb, value head hh) owns tokens
// bb*T .. bb*T+T-1 and blocks (bb*H + hh)*nt .. +nt-1.  Packed batches: the
// table k_varlen_plan writes, clamped offsets cu[B+1], first chunks
// first[B+1] (first[B] = the chunk count), then from word 2(B+1) one
// {first token, length} pair per chunk; chunk c of head hh owns block
// hh*ncmax + c.  Every per-chunk array (factors, checkpoints, exit
// gradients) is indexed by that block number.
// ---------------------------------------------------------------------------
struct ChainSpan {
    int64_t tok0;   // packed index of the sequence's first token
    int64_t tlen;   // its token count
    int64_t blk0;   // block of its first chunk
    int nt;         // its chunk count
};

__device__ inline ChainSpan chain_span(const int* plan, int64_t ncmax, int64_t B, int64_t T, int64_t H, int nt,
                                       int64_t bb, int64_t hh)
{
    if (plan == nullptr) return ChainSpan{bb * T, T, (bb * H + hh) * nt, nt};
    const int* first = plan + (B + 1);
    return ChainSpan{plan[bb], (int64_t)plan[bb + 1] - plan[bb], hh * ncmax + first[bb], first[bb + 1] - first[bb]};
}

// block ci of a launch with one workgroup per block: its value head, the
// packed index of its first token and its token count; false for the blocks
// of a packed batch past its last chunk
struct ChunkPos {
    int64_t hh, tok0;
    int len;
};

__device__ inline bool chunk_pos(const int* plan, int64_t ncmax, int64_t B, int64_t T, int64_t H, int nt, int64_t ci,
                                 ChunkPos& c)
{
    if (plan == nullptr) {
        const int64_t chain = ci / nt, bb = chain / H;
        const int64_t t0 = (ci - chain * nt) * (int64_t)kChunk;
        c.hh = chain - bb * H;
        c.tok0 = bb * T + t0;
        c.len = (int)(T - t0 < kChunk ? T - t0 : kChunk);
        return true;
    }
    c.hh = ci / ncmax;
    const int64_t gc = ci - c.hh * ncmax;
    if (gc >= plan[2 * B + 1]) return false;
    const int2 e = reinterpret_cast<const int2*>(plan + 2 * (B + 1))[gc];
    c.tok0 = e.x;
    c.len = e.y;
    return true;
}

}  // namespace gdn2
