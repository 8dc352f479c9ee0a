// Stand-ins for the device side of libgdn2, for a host-only build of the
// C-ABI layer (gdn2_api.cpp) under AddressSanitizer and UndefinedBehavior-
// Sanitizer: no GPU, no HIP runtime.
//
// "Device" buffers are ranges of an address-space reservation that is never
// readable (PROT_NONE), so a host dereference of a device pointer crashes.
// Every launch hook records the launch and checks that each pointer it is
// handed lies inside one registered buffer, and that the workspace blocks
// the launch will touch fit inside the workspace it was given.
#include "host_stubs.hpp"

#include <sys/mman.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#include "gdn2.h"
#include "gdn2_launch.hpp"

namespace {

struct Buf {
    uintptr_t lo, hi;
};

char* g_base = nullptr;
size_t g_used = 0;
constexpr size_t kReserve = size_t(1) << 36;   // 64 GiB of address space, none of it backed
std::vector<Buf> g_bufs;
int g_launches = 0;
int g_failures = 0;

void fail(const char* hook, const char* what)
{
    std::fprintf(stderr, "stub %s: %s\n", hook, what);
    ++g_failures;
}

// p (nullable unless required) lies in one buffer with `bytes` after it
void in_buf(const char* hook, const char* name, const void* p, int64_t bytes, bool required = false)
{
    if (p == nullptr) {
        if (required) fail(hook, name);
        return;
    }
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    for (const Buf& b : g_bufs)
        if (a >= b.lo && a < b.hi) {
            if (bytes > 0 && a + static_cast<uintptr_t>(bytes) > b.hi) fail(hook, name);
            return;
        }
    fail(hook, name);
}

}  // namespace

namespace stub {

void* dev_alloc(size_t bytes)
{
    if (g_base == nullptr) {
        void* m = mmap(nullptr, kReserve, PROT_NONE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1, 0);
        if (m == MAP_FAILED) {
            std::perror("mmap");
            std::abort();
        }
        g_base = static_cast<char*>(m);
    }
    const size_t n = (bytes + 255) / 256 * 256 + 256;   // 256-byte aligned, one granule apart
    if (g_used + n > kReserve) std::abort();
    char* p = g_base + g_used;
    g_used += n;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    g_bufs.push_back(Buf{lo, lo + bytes});
    return p;
}

void reset_launches() { g_launches = 0; }
int launches() { return g_launches; }
int failures() { return g_failures; }

}  // namespace stub

// ---- HIP runtime -----------------------------------------------------------
extern "C" hipError_t hipGetDevice(int* d)
{
    *d = 0;
    return hipSuccess;
}

// the side stream and events of the piecewise chunked forward: opaque handles
static int g_handles[64];
static int g_nhandles = 0;
extern "C" hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int)
{
    *s = reinterpret_cast<hipStream_t>(&g_handles[g_nhandles++ % 64]);
    return hipSuccess;
}
extern "C" hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned int)
{
    *e = reinterpret_cast<hipEvent_t>(&g_handles[g_nhandles++ % 64]);
    return hipSuccess;
}
extern "C" hipError_t hipEventRecord(hipEvent_t e, hipStream_t)
{
    return e != nullptr ? hipSuccess : hipErrorInvalidValue;
}
extern "C" hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* c)
{
    *c = hipStreamCaptureStatusNone;
    return hipSuccess;
}
extern "C" hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t e, unsigned int)   // null stream: the default one
{
    return e != nullptr ? hipSuccess : hipErrorInvalidValue;
}

// ---- launch hooks ----------------------------------------------------------
namespace gdn2 {

static int64_t prep_blocks(const PrepArgs& a) { return a.plan ? a.H * a.ncmax : a.B * a.H * a.nt; }

hipError_t launch_chunk_prep(const PrepArgs& a, int dk, bool bf16, bool gbf16, hipStream_t)
{
    ++g_launches;
    const char* h = "launch_chunk_prep";
    // whole extents of the token tensors (equal-length batches: B sequences of T)
    const int64_t es = bf16 ? 2 : 4, gs = gbf16 ? 2 : 4, tok = a.plan ? a.T : a.B * a.T;
    in_buf(h, "q", a.q, tok * a.Hk * dk * es, true);
    in_buf(h, "k", a.k, tok * a.Hk * dk * es, true);
    in_buf(h, "v", a.v, tok * a.H * a.dv * es, true);
    in_buf(h, "alpha", a.alpha, tok * a.H * dk * gs, true);
    in_buf(h, "b", a.b, tok * a.H * dk * gs, true);
    in_buf(h, "w", a.w, tok * a.H * a.dv * gs, true);
    in_buf(h, "workspace blocks", a.ws, prep_blocks(a) * a.ws_block, true);
    in_buf(h, "plan", a.plan, 0);
    if (a.conv_w != nullptr) {
        if (a.conv_K < 1 || a.conv_K > 4 || a.plan != nullptr) fail(h, "conv taps / packed batch");
        in_buf(h, "conv weight", a.conv_w, a.conv_C * a.conv_K * 4, true);
        in_buf(h, "conv window", a.conv_in, a.B * (a.conv_K - 1) * a.conv_C * 2);
    }
    return hipSuccess;
}

hipError_t launch_chunk_state(const StateArgs& a, int dk, int vs, bool bf16, hipStream_t)
{
    ++g_launches;
    const char* h = "launch_chunk_state";
    if (vs <= 0 || a.dv % vs != 0 || a.nslices * vs != a.dv) fail(h, "value slices");
    const int64_t nblk = a.plan ? a.H * a.ncmax : a.B * a.H * a.nt;
    const bool any = a.plan ? a.T > 0 : a.nt > 0;
    if (any) in_buf(h, "workspace blocks", a.ws, nblk * a.ws_block, true);
    in_buf(h, "plan", a.plan, 0);
    const int64_t st = a.B * a.H * dk * a.dv * 4;   // B counts sequences in a packed batch
    in_buf(h, "S0", a.S0, st);
    in_buf(h, "S_out", a.S_out, st);
    in_buf(h, "o", a.o, 0);
    // checkpoints: one [dk][dv] per workspace block
    in_buf(h, "S_chk", a.S_chk, nblk * dk * a.dv * 4);
    in_buf(h, "S_chkT", a.S_chkT, nblk * dk * a.dv * (bf16 ? 2 : 4));
    in_buf(h, "S_chkIo", a.S_chkIo, nblk * dk * a.dv * (bf16 ? 2 : 4));
    if (a.conv_out != nullptr) {
        for (const void* p : {a.cq, a.ck, a.cv}) in_buf(h, "conv input", p, 0, a.T > 0);   // read only at positions >= 0
        in_buf(h, "conv window in", a.conv_in, a.B * (a.conv_K - 1) * a.conv_C * 2);
        in_buf(h, "conv window out", a.conv_out, a.B * (a.conv_K - 1) * a.conv_C * 2, true);
    }
    return hipSuccess;
}

hipError_t launch_recurrent(const RecArgs& a, int dk, int vs, bool, bool, hipStream_t)
{
    ++g_launches;
    const char* h = "launch_recurrent";
    if (vs <= 0 || a.dv % vs != 0 || a.nslices * vs != a.dv) fail(h, "value slices");
    for (const void* p : {a.q, a.k, a.v, a.alpha, a.b, a.w}) in_buf(h, "input", p, 0, a.T > 0);
    const int64_t st = a.B * a.H * dk * a.dv * 4;
    in_buf(h, "S_in", a.S_in, st);
    in_buf(h, "S_out", a.S_out, st);
    in_buf(h, "o", a.o, 0);
    in_buf(h, "cu", a.cu, 4 * (a.B + 1));
    in_buf(h, "norm_g", a.norm_g, 0);
    in_buf(h, "norm_w", a.norm_w, 4 * a.dv);
    if (a.conv_w != nullptr) {
        in_buf(h, "conv weight", a.conv_w, a.conv_C * a.conv_K * 4, true);
        in_buf(h, "conv window in", a.conv_in, a.B * (a.conv_K - 1) * a.conv_C * 2);
        in_buf(h, "conv window out", a.conv_out, a.B * (a.conv_K - 1) * a.conv_C * 2);
    }
    return hipSuccess;
}

hipError_t launch_gated_rmsnorm(const NormArgs& a, bool bf16, hipStream_t)
{
    ++g_launches;
    const int64_t bytes = a.rows * a.dv * (bf16 ? 2 : 4);
    in_buf("launch_gated_rmsnorm", "o", a.o, bytes, true);
    in_buf("launch_gated_rmsnorm", "g", a.g, bytes, true);
    in_buf("launch_gated_rmsnorm", "y", a.y, bytes, true);
    in_buf("launch_gated_rmsnorm", "weight", a.weight, 4 * a.dv, true);
    return hipSuccess;
}

hipError_t launch_short_conv(const ConvArgs& a, int K, bool, bool bf16, hipStream_t)
{
    ++g_launches;
    const int64_t es = bf16 ? 2 : 4;
    in_buf("launch_short_conv", "x", a.x, a.B * a.T * a.C * es, true);
    in_buf("launch_short_conv", "y", a.y, a.B * a.T * a.C * es, true);
    in_buf("launch_short_conv", "weight", a.weight, a.C * K * 4, true);
    in_buf("launch_short_conv", "state_in", a.state_in, a.B * (K - 1) * a.C * es);
    in_buf("launch_short_conv", "state_out", a.state_out, a.B * (K - 1) * a.C * es);
    return hipSuccess;
}

hipError_t launch_short_conv_bwd(const ConvBwdArgs& a, int K, bool, bool bf16, hipStream_t)
{
    ++g_launches;
    const int64_t es = bf16 ? 2 : 4;
    const char* h = "launch_short_conv_bwd";
    in_buf(h, "x", a.x, a.B * a.T * a.C * es, true);
    in_buf(h, "dy", a.dy, a.B * a.T * a.C * es, true);
    in_buf(h, "dx", a.dx, a.B * a.T * a.C * es, true);
    in_buf(h, "weight", a.weight, a.C * K * 4, true);
    in_buf(h, "dweight", a.dweight, a.C * K * 4, true);
    in_buf(h, "state_in", a.state_in, a.B * (K - 1) * a.C * es);
    in_buf(h, "dstate", a.dstate, a.B * (K - 1) * a.C * es);
    in_buf(h, "dstate_out", a.dstate_out, a.B * (K - 1) * a.C * es);
    in_buf(h, "partials", a.part, a.B * a.nspan * a.C * K * 4, true);
    return hipSuccess;
}

hipError_t launch_varlen_plan(const PlanArgs& a, hipStream_t)
{
    ++g_launches;
    in_buf("launch_varlen_plan", "cu", a.cu, 4 * (a.N + 1), true);
    in_buf("launch_varlen_plan", "plan", a.plan, 4 * plan_head_words(a.N) + 8 * a.ncmax, true);
    return hipSuccess;
}

hipError_t launch_chunk_state_bwd(const BwdStateArgs& a, bool bf16, hipStream_t)
{
    ++g_launches;
    const char* h = "launch_chunk_state_bwd";
    const int64_t nblk = a.plan ? a.H * a.ncmax : a.B * a.H * a.nt;
    const bool any = a.plan ? a.T > 0 : a.nt > 0;
    if (a.plan != nullptr && a.nt != 0) fail(h, "chunk count with a plan");
    in_buf(h, "plan", a.plan, 4 * plan_head_words(a.B) + 8 * a.ncmax);
    in_buf(h, "workspace blocks", a.ws, nblk * a.ws_block, any);
    in_buf(h, "dO", a.dO, 0, any);
    in_buf(h, "dSL", a.dSL, nblk * a.dk * a.dv * 4);
    in_buf(h, "dSLIo", a.dSLIo, nblk * a.dk * a.dv * (bf16 ? 2 : 4));
    in_buf(h, "dSLT", a.dSLT, nblk * a.dk * a.dv * (bf16 ? 2 : 4));
    in_buf(h, "dS0", a.dS0, a.B * a.H * a.dk * a.dv * 4);
    in_buf(h, "dS_T", a.dS_T, a.B * a.H * a.dk * a.dv * 4);
    return hipSuccess;
}

hipError_t launch_chunk_state_bwd_mf(const BwdStateArgs& a, hipStream_t s) { return launch_chunk_state_bwd(a, true, s); }

int state_bwd_slice(int dv) { return dv % 16 == 0 ? 16 : 0; }

hipError_t launch_bwd_qk_map(const QkMapArgs& a, bool post, bool bf16, hipStream_t)
{
    ++g_launches;
    const int64_t es = bf16 ? 2 : 4, src = a.rows * a.dk * es, dst = src * a.G;
    const char* h = "launch_bwd_qk_map";
    in_buf(h, "q", a.q, src, true);
    in_buf(h, "k", a.k, src, true);
    if (post) {
        in_buf(h, "dqh", a.dqh, dst, true);
        in_buf(h, "dkh", a.dkh, dst, true);
        in_buf(h, "dq", a.dq, src, true);
        in_buf(h, "dk", a.dk_out, src, true);
    } else {
        in_buf(h, "qh", a.qh, dst, true);
        in_buf(h, "kh", a.kh, dst, true);
    }
    return hipSuccess;
}

hipError_t launch_bwd_gate_map(const GateMapArgs& a, bool post, bool gbf16, hipStream_t)
{
    ++g_launches;
    for (int j = 0; j < 3; ++j) {
        in_buf("launch_bwd_gate_map", "z", a.z[j], a.n[j] * (gbf16 ? 2 : 4), true);
        in_buf("launch_bwd_gate_map", "dst", a.dst[j], a.n[j] * (post ? (gbf16 ? 2 : 4) : 4), true);
        if (post) in_buf("launch_bwd_gate_map", "grad", a.grad[j], a.n[j] * 4, true);
    }
    return hipSuccess;
}

hipError_t launch_chunk_grad(const GradArgs& a, bool, bool, hipStream_t)
{
    ++g_launches;
    const char* h = "launch_chunk_grad";
    for (const void* p : {a.q, a.k, a.v, a.alpha, a.b, a.w, a.dO}) in_buf(h, "input", p, 0, true);
    for (void* p : {a.dq, a.dk_out, a.dv_out, a.dalpha, a.db, a.dw}) in_buf(h, "output", p, 0, true);
    if (a.total != (a.plan ? a.H * a.ncmax : a.B * a.H * a.nt)) fail(h, "block count");
    in_buf(h, "plan", a.plan, 4 * plan_head_words(a.B) + 8 * a.ncmax);
    in_buf(h, "S_chk", a.S_chk, a.total * a.dk * a.dv * 4, true);
    in_buf(h, "dSL", a.dSL, a.total * a.dk * a.dv * 4, true);
    in_buf(h, "scratch", a.scratch, chunk_grad_scratch_bytes(a.dk, a.dv, a.total), true);
    return hipSuccess;
}

hipError_t launch_chunk_grad_mf(const GradVArgs& v, const GradKArgs& k, bool, hipStream_t)
{
    ++g_launches;
    const char* h = "launch_chunk_grad_mf";
    if (v.total != (v.plan ? v.H * v.ncmax : v.B * v.H * v.nt) || k.total != v.total || k.plan != v.plan ||
        k.ncmax != v.ncmax)
        fail(h, "block count");
    in_buf(h, "plan", v.plan, 4 * plan_head_words(v.B) + 8 * v.ncmax);
    in_buf(h, "workspace blocks", v.ws, v.total * v.ws_block, true);
    for (const void* p : {v.S_chk, v.S_chkT, v.dSL, v.dSLT}) in_buf(h, "checkpoint", p, v.total * v.dk * v.dv * 2, true);
    for (const void* p : {v.v, v.w, v.dO}) in_buf(h, "input", p, 0, true);
    for (const void* p : {k.q, k.k, k.alpha, k.b}) in_buf(h, "input", p, 0, true);
    for (void* p : {v.dw, v.dv_out, k.dq, k.dk_out, k.dalpha, k.db}) in_buf(h, "output", p, 0, true);
    return hipSuccess;
}

bool gradmf_supported(int dk, int dv, bool bf16)
{
    return bf16 && (dk == 32 || dk == 64 || dk == 128) && (dv == 32 || dv == 64 || dv == 128);
}

int64_t grad_blocks(int64_t total) { return total < 1024 ? total : 1024; }
int64_t chunk_grad_scratch_bytes(int dk, int dv, int64_t total) { return grad_blocks(total) * (dk * dv + 4096) * 4; }

void* noalloc_scratch()
{
    static void* p = stub::dev_alloc(GDN2_NOALLOC_SCRATCH_BYTES);
    return p;
}

int chunk_state_slice(int64_t, int dv, int, int)
{
    for (int w : {64, 32, 16})
        if (dv % w == 0) return w;
    return 16;
}

int recurrent_slice(int64_t, int64_t T, int dv)
{
    for (int w : {128, 64, 32, 16})
        if (dv % w == 0 && (T <= 1 || w <= 64)) return w;
    return 16;
}

}  // namespace gdn2
