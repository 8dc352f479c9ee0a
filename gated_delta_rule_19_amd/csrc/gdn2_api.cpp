// C ABI of the GDN-2 token-mixer core (include/gdn2.h): argument checks on
// the host, workspace sizing, and the kernel launches on the caller's stream.
//
// Everything that can be decided from the arguments is checked before the
// first HIP call, so an invalid call never touches the device.  No function
// here allocates, frees or synchronises.
#include "gdn2.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "gdn2_launch.hpp"
#include "gdn2_layout.hpp"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 40;   // larger sizes are rejected as shape errors

struct Range {
    uintptr_t lo, hi;   // [lo, hi); empty when lo == hi
};

Range range_of(const void* p, int64_t bytes)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, (p != nullptr && bytes > 0) ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool overlap(Range a, Range b)
{
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// checks shared by every entry point; `chunked` adds the chunk-length rule,
// `varlen` reads B as the sequence count and T as the packed token count
int check_problem(const gdn2_problem* p, bool chunked, bool varlen = false)
{
    if (p == nullptr) return GDN2_ERR_NULL;
    if (p->B < 0 || p->T < 0 || p->H < 0 || p->B > kMaxDim || p->T > kMaxDim || p->H > kMaxDim)
        return GDN2_ERR_SHAPE;
    if (p->Hv < 0 || p->Hv > kMaxDim) return GDN2_ERR_SHAPE;
    if (p->Hv != 0 && (p->H == 0 || p->Hv % p->H != 0)) return GDN2_ERR_SHAPE;
    if (!(p->dk == 16 || p->dk == 32 || p->dk == 64 || p->dk == 128)) return GDN2_ERR_SHAPE;
    if (p->dv < 16 || p->dv > 256 || p->dv % 16 != 0) return GDN2_ERR_SHAPE;
    if (chunked && p->chunk != 64) return GDN2_ERR_SHAPE;
    if ((p->flags & ~(GDN2_FLAG_GATE_LOGITS | GDN2_FLAG_NEG_EIGVAL | GDN2_FLAG_QK_L2NORM)) != 0)
        return GDN2_ERR_SHAPE;
    if ((p->flags & GDN2_FLAG_NEG_EIGVAL) && !(p->flags & GDN2_FLAG_GATE_LOGITS)) return GDN2_ERR_SHAPE;
    // element counts stay far inside int64 and every grid inside 2^31 workgroups
    const double hv = double(p->Hv != 0 ? p->Hv : p->H);
    if (!varlen) {
        const double rows = double(p->B) * double(p->T) * hv;
        if (rows * 256.0 > 9.0e15) return GDN2_ERR_SHAPE;
        if (double(p->B) * hv * (double((p->T + 63) / 64) + 16.0) > 2.0e9) return GDN2_ERR_SHAPE;
    } else {
        // int32 token offsets; prep grid hv * (ceil(T/64) + N), state grid N * hv * slices
        if (p->T > INT32_MAX - 64 || p->B > INT32_MAX / 4) return GDN2_ERR_SHAPE;
        if (double(p->T) * hv * 256.0 > 9.0e15) return GDN2_ERR_SHAPE;
        if (hv * (double((p->T + 63) / 64) + double(p->B)) > 2.0e9) return GDN2_ERR_SHAPE;
        if (double(p->B) * hv * 16.0 > 2.0e9) return GDN2_ERR_SHAPE;
    }
    const bool f32 = p->io_dtype == GDN2_F32 && p->gate_dtype == GDN2_F32;
    const bool bf = p->io_dtype == GDN2_BF16 && (p->gate_dtype == GDN2_F32 || p->gate_dtype == GDN2_BF16);
    if (!f32 && !bf) return GDN2_ERR_DTYPE;
    return GDN2_OK;
}

bool is_bf16(const gdn2_problem* p) { return p->io_dtype == GDN2_BF16; }
// value heads: each has its own state, gates and values (q and k are per query/key head)
int64_t nvh(const gdn2_problem* p) { return p->Hv != 0 ? p->Hv : p->H; }
bool gates_bf16(const gdn2_problem* p) { return p->gate_dtype == GDN2_BF16; }
int64_t gate_size(const gdn2_problem* p) { return gates_bf16(p) ? 2 : 4; }
int64_t io_size(const gdn2_problem* p) { return is_bf16(p) ? 2 : 4; }
int64_t nchunks(const gdn2_problem* p) { return (p->T + 63) / 64; }

int64_t ws_block_bytes(const gdn2_problem* p)
{
    return gdn2::ws_layout(p->dk, p->dv, io_size(p), is_bf16(p) ? 32 : 16).block;
}

int64_t ws_bytes(const gdn2_problem* p) { return p->B * nvh(p) * nchunks(p) * ws_block_bytes(p); }

// workspace gdn2_chunk_fwd needs: the two stages' factor blocks
int64_t fwd_ws_bytes(const gdn2_problem* p) { return ws_bytes(p); }

// packed batches: the chunk plan, then one block per (value head, chunk slot)
int64_t varlen_ncmax(const gdn2_problem* p) { return nchunks(p) + p->B; }
int64_t varlen_plan_bytes(const gdn2_problem* p)
{
    return (4 * gdn2::plan_head_words(p->B) + 8 * varlen_ncmax(p) + 255) / 256 * 256;
}
int64_t varlen_ws_bytes(const gdn2_problem* p)
{
    return varlen_plan_bytes(p) + nvh(p) * varlen_ncmax(p) * ws_block_bytes(p);
}

struct Sizes {
    int64_t key, val, state;   // bytes of q or k [B,T,H,dk], of v or o [B,T,Hv,dv], of a state
    int64_t gk, gv;            // bytes of alpha or b [B,T,Hv,dk], of w [B,T,Hv,dv]
};

// token tensors span B sequences of T tokens, or (varlen) T packed tokens
Sizes sizes_of(const gdn2_problem* p, bool varlen = false)
{
    const int64_t tok = varlen ? p->T : p->B * p->T;
    const int64_t rows = tok * p->H, vrows = tok * nvh(p);
    return Sizes{rows * p->dk * io_size(p), vrows * p->dv * io_size(p), p->B * nvh(p) * p->dk * p->dv * 4,
                 vrows * p->dk * gate_size(p), vrows * p->dv * gate_size(p)};
}

bool rows_nonempty(const gdn2_problem* p) { return p->B * p->T * p->H > 0; }

// inputs must be non-null whenever they hold any element (a packed batch of
// B > 0 sequences holds T tokens)
int check_inputs(const gdn2_problem* p, const void* q, const void* k, const void* v,
                 const void* alpha, const void* b, const void* w, const void* o)
{
    if (!rows_nonempty(p)) return GDN2_OK;
    if (!q || !k || !v || !alpha || !b || !w || !o) return GDN2_ERR_NULL;
    return GDN2_OK;
}

// outputs may not overlap inputs or each other; the state may be updated in
// place only when the pointers are identical
int check_alias(const Range* outs, int nout, const Range* ins, int nin, const void* s_in, const void* s_out,
                int s_in_idx, int s_out_idx)
{
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j) {
            if (i == s_out_idx && j == s_in_idx && s_in == s_out) continue;
            if (overlap(outs[i], ins[j])) return GDN2_ERR_ALIAS;
        }
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j])) return GDN2_ERR_ALIAS;
    }
    return GDN2_OK;
}

// the offsets of a packed batch: present, int32-aligned
int check_cu(const gdn2_problem* p, const int32_t* cu)
{
    if (p->B * nvh(p) == 0) return GDN2_OK;
    if (cu == nullptr) return GDN2_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(cu) & 3u) != 0) return GDN2_ERR_ALIGN;
    return GDN2_OK;
}

int check_align(std::initializer_list<const void*> ptrs)
{
    for (const void* p : ptrs)
        if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return GDN2_ERR_ALIGN;
    return GDN2_OK;
}

int device_ready()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GDN2_ERR_DEVICE;
    return GDN2_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? GDN2_OK : GDN2_ERR_DEVICE; }

// channels of the fused short convolution: q | k | v of the concatenated projection
int64_t conv_channels(const gdn2_problem* p) { return 2 * p->H * p->dk + nvh(p) * p->dv; }

// the fused convolution's window moves only when it has taps before the
// current token and somewhere new to go
bool conv_window_moves(const gdn2_conv* c)
{
    return c != nullptr && c->K > 1 && c->state_out != nullptr && c->state_out != c->state_in;
}

int do_prep(const gdn2_problem* p, const void* q, const void* k, const void* v, const void* alpha,
            const void* b, const void* w, void* ws, hipStream_t s, const gdn2_conv* conv = nullptr)
{
    if (p->B * nvh(p) * nchunks(p) == 0) return GDN2_OK;
    gdn2::PrepArgs a{q, k, v, alpha, b, w, ws, ws_block_bytes(p), p->B, p->T, nvh(p), p->H,
                     (int)p->dv, (int)nchunks(p), (int)p->flags, nullptr, 0};
    if (conv != nullptr) {
        a.conv_w = conv->weight;
        a.conv_in = conv->K > 1 ? conv->state_in : nullptr;
        a.conv_C = conv_channels(p);
        a.conv_K = conv->K;
        a.conv_silu = (conv->flags & GDN2_CONV_SILU) != 0;
    }
    return launch_status(gdn2::launch_chunk_prep(a, (int)p->dk, is_bf16(p), gates_bf16(p), s));
}

// conv (optional): the fused convolution whose window after the last token
// the first slice of each chain writes (q, k, v: the raw inputs)
int do_state(const gdn2_problem* p, const float* S0, void* o, float* S_out, const void* ws, hipStream_t s,
             const gdn2_conv* conv = nullptr, const void* q = nullptr, const void* k = nullptr,
             const void* v = nullptr)
{
    const int64_t nch = p->B * nvh(p);
    if (nch == 0) return GDN2_OK;
    const bool window = conv != nullptr && conv->K > 1 && conv->state_out != nullptr;
    if (nchunks(p) == 0 && S_out == S0 && !conv_window_moves(conv)) return GDN2_OK;   // nothing to do
    const int vs = gdn2::chunk_state_slice(nch, (int)p->dv, (int)p->dk, (int)io_size(p));
    gdn2::StateArgs a{ws, ws_block_bytes(p), S0, o, S_out, p->B, p->T, nvh(p), (int)p->dv,
                      (int)nchunks(p), (int)(p->dv / vs), nullptr, 0};
    if (window) {
        a.cq = q;
        a.ck = k;
        a.cv = v;
        a.conv_in = conv->state_in;
        a.conv_out = conv->state_out;
        a.conv_C = conv_channels(p);
        a.Hk = p->H;
        a.conv_K = conv->K;
    }
    return launch_status(gdn2::launch_chunk_state(a, (int)p->dk, vs, is_bf16(p), s));
}

// the fused convolution's descriptor: taps, option, weights present and
// aligned; equal-length batches only
int check_conv(const gdn2_problem* p, const gdn2_conv* c)
{
    if (c == nullptr || c->weight == nullptr) return GDN2_ERR_NULL;
    if (c->K < 1 || c->K > 4) return GDN2_ERR_SHAPE;
    if (c->flags != 0 && c->flags != GDN2_CONV_SILU) return GDN2_ERR_SHAPE;
    (void)p;
    return GDN2_OK;
}

// ranges of the convolution's weights and windows
Range conv_weight_range(const gdn2_problem* p, const gdn2_conv* c)
{
    return range_of(c->weight, conv_channels(p) * c->K * 4);
}
Range conv_state_range(const gdn2_problem* p, const gdn2_conv* c, const void* ptr)
{
    return range_of(c->K > 1 ? ptr : nullptr, p->B * (c->K - 1) * conv_channels(p) * io_size(p));
}

// backward workspace: forward factors | chunk entry states | chunk exit
// state gradients | gradient scratch, each 256-byte aligned.  The vector-ALU
// path keeps both checkpoints in fp32 [dk][dv]; the matrix-core path (bf16
// I/O, dk and dv in {32, 64, 128}) keeps the backward's extension in each
// factor block, both checkpoints in bf16, [dk][dv] and transposed [dv][dk]
// (its products take bf16 operands, so an fp32 copy would only be rounded
// again), and needs no gradient scratch (its two gradient stages share LDS).
struct BwdLayout {
    bool mf;
    int64_t block, t_off;                 // factor block stride, offset of T in it
    int64_t blk;                          // offset of the first factor block
    int64_t chk, chkT, dsl, dslT, scratch, total;
};

// nblk: the factor blocks (B*H*nchunks, or H*ncmax for a packed batch)
BwdLayout bwd_layout(const gdn2_problem* p, int64_t nblk)
{
    const int64_t states = nblk * p->dk * p->dv * 4;
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    BwdLayout l{};
    l.mf = gdn2::gradmf_supported((int)p->dk, (int)p->dv, is_bf16(p));
    l.block = ws_block_bytes(p);
    if (l.mf) {                           // the backward's layout of the blocks (BwdExt)
        l.t_off = l.block;
        l.block = gdn2::bwd_ext(l.block, p->dk).block;
    }
    const int64_t chk = l.mf ? states / 2 : states;        // one copy of one checkpoint set
    l.chk = up(nblk * l.block);
    l.chkT = up(l.chk + chk);
    l.dsl = l.mf ? up(l.chkT + chk) : l.chkT;
    l.dslT = up(l.dsl + chk);
    l.scratch = l.mf ? up(l.dslT + chk) : l.dslT;
    l.total = l.scratch + (l.mf ? 0 : gdn2::chunk_grad_scratch_bytes((int)p->dk, (int)p->dv, nblk));
    return l;
}

// Prologue options and shared query/key heads in the backward: the core runs
// with no flags and one query/key row per value head on inputs materialised in
// workspace after its own (activated gates as fp32; q/k rows normalised and
// widened to the value heads), and its gradients of those are mapped back.
// A packed batch (varlen: B sequences, T packed tokens) puts its chunk plan
// first and gives every value head ncmax blocks.
struct BwdWrap {
    gdn2_problem core;     // the problem the core backward sees
    BwdLayout l;           // its workspace layout, from `base` on
    bool qk, gates;        // q/k rows materialised; gates activated
    int64_t base;          // bytes of the chunk plan ahead of the layout (0: equal lengths)
    int64_t ncmax;         // block slots per value head (packed batches)
    int64_t tok;           // token rows of the tensors: B*T, or T packed
    int64_t qh, kh, dqh, dkh, ga, gb, gw, dga, dgb, dgw, total;
};

BwdWrap bwd_wrap(const gdn2_problem* p, bool varlen = false)
{
    BwdWrap w{};
    w.core = *p;
    w.base = varlen ? varlen_plan_bytes(p) : 0;
    w.ncmax = varlen ? varlen_ncmax(p) : 0;
    w.tok = varlen ? p->T : p->B * p->T;
    auto blocks = [&](const gdn2_problem* c) { return varlen ? c->H * w.ncmax : c->B * c->H * nchunks(c); };
    auto shift = [&](BwdLayout l) {       // the layout's offsets from the start of the workspace
        l.blk += w.base; l.chk += w.base; l.chkT += w.base; l.dsl += w.base; l.dslT += w.base;
        l.scratch += w.base; l.total += w.base;
        return l;
    };
    w.l = shift(bwd_layout(p, blocks(p)));
    // the matrix-core kernels apply the prologue options themselves; shared
    // query/key heads still need q/k widened to the value heads (and their
    // gradients summed per group, through the norm when it is on), and the
    // vector-ALU path needs every mapping
    const bool mf = w.l.mf;
    if (mf && nvh(p) == p->H) {
        w.core.Hv = 0;
        w.total = w.l.total;
        return w;
    }
    w.qk = (p->flags & GDN2_FLAG_QK_L2NORM) != 0 || nvh(p) != p->H;
    w.gates = !mf && (p->flags & GDN2_FLAG_GATE_LOGITS) != 0;
    w.core.flags = mf ? (p->flags & ~GDN2_FLAG_QK_L2NORM) : 0;   // gate options stay in-kernel
    w.core.H = nvh(p);
    w.core.Hv = 0;
    if (w.gates) w.core.gate_dtype = GDN2_F32;
    w.l = shift(bwd_layout(&w.core, blocks(&w.core)));
    int64_t off = w.l.total;
    auto take = [&off](int64_t bytes) {
        const int64_t o = (off + 255) & ~int64_t(255);
        off = o + bytes;
        return o;
    };
    const int64_t vrows = w.tok * nvh(p);
    if (w.qk) {
        const int64_t bytes = vrows * p->dk * io_size(p);
        w.qh = take(bytes); w.kh = take(bytes); w.dqh = take(bytes); w.dkh = take(bytes);
    }
    if (w.gates) {
        const int64_t gk = vrows * p->dk * 4, gv = vrows * p->dv * 4;
        w.ga = take(gk); w.gb = take(gk); w.gw = take(gv);
        w.dga = take(gk); w.dgb = take(gk); w.dgw = take(gv);
    }
    w.total = off;
    return w;
}

// the core backward: H value heads = query/key heads; prologue flags only on
// the matrix-core path.  plan (null for equal-length batches): the packed
// batch's chunk plan, already written, with ncmax block slots per head.
int bwd_core(const gdn2_problem* p, const BwdLayout& l, const int* plan, int64_t ncmax, const void* q,
             const void* k, const void* v, const void* alpha, const void* b, const void* w, const float* S0,
             const void* dO, const float* dS_T, void* dq, void* dk, void* dv, void* dalpha, void* db, void* dw,
             float* dS0, char* ws, hipStream_t s)
{
    int st = GDN2_OK;
    char* blocks = ws + l.blk;
    float* chk = l.mf ? nullptr : reinterpret_cast<float*>(ws + l.chk);     // fp32 checkpoints
    float* dsl = l.mf ? nullptr : reinterpret_cast<float*>(ws + l.dsl);
    void* chkIo = l.mf ? ws + l.chk : nullptr;                                // bf16, both layouts
    void* dslIo = l.mf ? ws + l.dsl : nullptr;
    void* chkT = l.mf ? ws + l.chkT : nullptr;
    void* dslT = l.mf ? ws + l.dslT : nullptr;
    const int64_t nch = p->B * p->H;
    const int nt = plan ? 0 : (int)nchunks(p);               // per chain; a plan gives each its own
    const int64_t total = plan ? p->H * ncmax : nch * nchunks(p);   // block slots
    if (p->flags != 0 && !l.mf) return GDN2_ERR_SHAPE;   // never reached: the mappings clear the flags
    if (nchunks(p) > 0) {
        gdn2::PrepArgs pa{q, k, v, alpha, b, w, blocks, l.block, p->B, p->T, p->H, p->H,
                          (int)p->dv, nt, (int)p->flags, plan, ncmax, l.t_off};
        st = launch_status(gdn2::launch_chunk_prep(pa, (int)p->dk, is_bf16(p), gates_bf16(p), s));
        if (st) return st;
        const int vs = gdn2::chunk_state_slice(nch, (int)p->dv, (int)p->dk, (int)io_size(p));
        gdn2::StateArgs fa{blocks, l.block, S0, nullptr, nullptr, p->B, p->T, p->H, (int)p->dv,
                           nt, (int)(p->dv / vs), plan, ncmax, chk, chkT, chkIo};
        st = launch_status(gdn2::launch_chunk_state(fa, (int)p->dk, vs, is_bf16(p), s));
        if (st) return st;
    }
    const int bvs = l.mf ? 32 : gdn2::state_bwd_slice((int)p->dv);
    gdn2::BwdStateArgs ba{blocks, l.block, dO, dS_T, dsl, dS0, p->B, p->T, p->H, (int)p->dk, (int)p->dv,
                          nt, (int)(p->dv / bvs), bvs, dslT, dslIo, l.t_off, plan, ncmax};
    st = launch_status(l.mf ? gdn2::launch_chunk_state_bwd_mf(ba, s) : gdn2::launch_chunk_state_bwd(ba, is_bf16(p), s));
    if (st) return st;
    if (nchunks(p) == 0) return GDN2_OK;
    float* gsc = reinterpret_cast<float*>(ws + l.scratch);
    if (l.mf) {
        gdn2::GradVArgs va{blocks, l.block, l.t_off, v, w, dO, chkIo, chkT, dslIo, dslT, dw, dv,
                           p->B, p->T, p->H, (int)p->dk, (int)p->dv, nt, total, (int)p->flags, plan, ncmax};
        gdn2::GradKArgs ka{q, k, alpha, b, dq, dk, dalpha, db, p->B, p->T, p->H, (int)p->dk,
                           nt, total, (int)p->flags, plan, ncmax};
        return launch_status(gdn2::launch_chunk_grad_mf(va, ka, gates_bf16(p), s));
    }
    gdn2::GradArgs ga{q, k, v, alpha, b, w, dO, chk, dsl, dq, dk, dv, dalpha, db, dw, gsc, p->B, p->T, p->H,
                      (int)p->dk, (int)p->dv, nt, total, plan, ncmax};
    return launch_status(gdn2::launch_chunk_grad(ga, is_bf16(p), gates_bf16(p), s));
}

// The backward once every argument has passed its checks: the prologue
// mappings (kernels over the token rows, wr.tok of them) around the core.
// A packed batch's plan is written first, into the workspace's head.
int bwd_run(const gdn2_problem* p, const BwdWrap& wr, const int32_t* cu_seqlens, const void* q, const void* k,
            const void* v, const void* alpha, const void* b, const void* w, const float* S0, const void* dO,
            const float* dS_T, void* dq, void* dk, void* dv, void* dalpha, void* db, void* dw, float* dS0,
            char* ws, hipStream_t s)
{
    int st = GDN2_OK;
    const int* plan = nullptr;
    if (cu_seqlens != nullptr) {
        int* pl = reinterpret_cast<int*>(ws);
        st = launch_status(gdn2::launch_varlen_plan(gdn2::PlanArgs{cu_seqlens, pl, p->B, p->T, wr.ncmax}, s));
        if (st) return st;
        plan = pl;
    }
    if (nchunks(p) == 0 || (!wr.qk && !wr.gates))   // no token to map: the core alone
        return bwd_core(&wr.core, wr.l, plan, wr.ncmax, q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk, dv, dalpha,
                        db, dw, dS0, ws, s);
    const void *cq = q, *ck = k, *ca = alpha, *cb = b, *cw = w;
    void *cdq = dq, *cdk = dk, *cda = dalpha, *cdb = db, *cdw = dw;
    const int G = (int)(nvh(p) / p->H);
    const gdn2::QkMapArgs qa{q, k, ws + wr.qh, ws + wr.kh, ws + wr.dqh, ws + wr.dkh, dq, dk,
                             wr.tok * p->H, G, (int)p->dk, (p->flags & GDN2_FLAG_QK_L2NORM) != 0};
    if (wr.qk) {
        st = launch_status(gdn2::launch_bwd_qk_map(qa, false, is_bf16(p), s));
        if (st) return st;
        cq = ws + wr.qh; ck = ws + wr.kh; cdq = ws + wr.dqh; cdk = ws + wr.dkh;
    }
    const int64_t vrows = wr.tok * nvh(p);
    const float bscale = (p->flags & GDN2_FLAG_NEG_EIGVAL) ? 2.f : 1.f;
    float* ga[3] = {reinterpret_cast<float*>(ws + wr.ga), reinterpret_cast<float*>(ws + wr.gb),
                    reinterpret_cast<float*>(ws + wr.gw)};
    float* dga[3] = {reinterpret_cast<float*>(ws + wr.dga), reinterpret_cast<float*>(ws + wr.dgb),
                     reinterpret_cast<float*>(ws + wr.dgw)};
    if (wr.gates) {
        const gdn2::GateMapArgs pre{{alpha, b, w}, {nullptr, nullptr, nullptr}, {ga[0], ga[1], ga[2]},
                                    {vrows * p->dk, vrows * p->dk, vrows * p->dv}, {1.f, bscale, 1.f}};
        st = launch_status(gdn2::launch_bwd_gate_map(pre, false, gates_bf16(p), s));
        if (st) return st;
        ca = ga[0]; cb = ga[1]; cw = ga[2];
        cda = dga[0]; cdb = dga[1]; cdw = dga[2];
    }
    st = bwd_core(&wr.core, wr.l, plan, wr.ncmax, cq, ck, v, ca, cb, cw, S0, dO, dS_T, cdq, cdk, dv, cda, cdb,
                  cdw, dS0, ws, s);
    if (st) return st;
    if (wr.qk) {
        st = launch_status(gdn2::launch_bwd_qk_map(qa, true, is_bf16(p), s));
        if (st) return st;
    }
    if (wr.gates) {
        const gdn2::GateMapArgs post{{alpha, b, w}, {dga[0], dga[1], dga[2]}, {dalpha, db, dw},
                                     {vrows * p->dk, vrows * p->dk, vrows * p->dv}, {1.f, bscale, 1.f}};
        st = launch_status(gdn2::launch_bwd_gate_map(post, true, gates_bf16(p), s));
    }
    return st;
}

}  // namespace

extern "C" {

int gdn2_abi_version(void) { return GDN2_ABI_VERSION; }

const char* gdn2_status_str(int status)
{
    switch (status) {
        case GDN2_OK: return "GDN2_OK: success";
        case GDN2_ERR_NULL: return "GDN2_ERR_NULL: a required pointer is NULL";
        case GDN2_ERR_SHAPE: return "GDN2_ERR_SHAPE: unsupported or inconsistent sizes";
        case GDN2_ERR_DTYPE: return "GDN2_ERR_DTYPE: unsupported dtype pair";
        case GDN2_ERR_ALIAS: return "GDN2_ERR_ALIAS: an output overlaps an input or another output";
        case GDN2_ERR_WORKSPACE: return "GDN2_ERR_WORKSPACE: workspace missing or too small";
        case GDN2_ERR_DEVICE: return "GDN2_ERR_DEVICE: no usable GPU or a launch failed";
        case GDN2_ERR_ALIGN: return "GDN2_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
        default: return "GDN2: unknown status";
    }
}

size_t gdn2_chunk_fwd_workspace_size(const gdn2_problem* p)
{
    if (check_problem(p, true) != GDN2_OK) return 0;
    return static_cast<size_t>(fwd_ws_bytes(p));
}

size_t gdn2_chunk_prep_workspace_size(const gdn2_problem* p)
{
    if (check_problem(p, true) != GDN2_OK) return 0;
    return static_cast<size_t>(ws_bytes(p));
}

int gdn2_chunk_prep(const gdn2_problem* p, const void* q, const void* k, const void* v,
                    const void* alpha, const void* b, const void* w, void* workspace,
                    size_t workspace_bytes, void* stream)
{
    int st = check_problem(p, true);
    if (st) return st;
    // the prep stage has no o; check inputs with a stand-in non-null output
    st = check_inputs(p, q, k, v, alpha, b, w, q);
    if (st) return st;
    const int64_t need = ws_bytes(p);
    if (need > 0 && (workspace == nullptr || static_cast<int64_t>(workspace_bytes) < need))
        return GDN2_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_WORKSPACE;
    const Sizes z = sizes_of(p);
    const Range ins[6] = {range_of(q, z.key), range_of(k, z.key), range_of(v, z.val),
                          range_of(alpha, z.gk), range_of(b, z.gk), range_of(w, z.gv)};
    const Range outs[1] = {range_of(workspace, need)};
    st = check_alias(outs, 1, ins, 6, nullptr, nullptr, -1, -1);
    if (st) return st;
    st = check_align({q, k, v, alpha, b, w});
    if (st) return st;
    if (need == 0) return GDN2_OK;
    st = device_ready();
    if (st) return st;
    return do_prep(p, q, k, v, alpha, b, w, workspace, static_cast<hipStream_t>(stream));
}

int gdn2_chunk_state(const gdn2_problem* p, const float* S0, void* o, float* S_out,
                     const void* workspace, size_t workspace_bytes, void* stream)
{
    int st = check_problem(p, true);
    if (st) return st;
    if (rows_nonempty(p) && o == nullptr) return GDN2_ERR_NULL;
    const int64_t need = ws_bytes(p);
    if (need > 0 && (workspace == nullptr || static_cast<int64_t>(workspace_bytes) < need))
        return GDN2_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_WORKSPACE;
    const Sizes z = sizes_of(p);
    const Range ins[2] = {range_of(workspace, need), range_of(S0, z.state)};
    const Range outs[2] = {range_of(o, z.val), range_of(S_out, z.state)};
    st = check_alias(outs, 2, ins, 2, S0, S_out, 1, 1);
    if (st) return st;
    st = check_align({S0, o, S_out});
    if (st) return st;
    if (p->B * p->H == 0 || (nchunks(p) == 0 && S_out == S0)) return GDN2_OK;
    st = device_ready();
    if (st) return st;
    return do_state(p, S0, o, S_out, workspace, static_cast<hipStream_t>(stream));
}

// ---- long single sequences: the prep of the next piece beside the state pass
// With few chains the serial state pass holds at most half of the CUs (one
// workgroup each) for a long time while the rest idle.  The sequence is then
// cut into pieces of whole chunks: piece i's state pass runs on the caller's
// stream while the preps of the pieces after it run on a second stream on
// the other CUs.  Each piece has its own part of the workspace (the same
// bytes in all), the state is carried through S_out, and the pieces are
// ordered only by events (no workgroup waits for another).  Pieces are 32
// chunks long: at 16 chains a piece's factors (37 MB) then stay in the
// last-level cache beside the next pieces' preps (B1 H16 T65536: 1,540 us a
// call against 1,860 with pieces of 128 chunks, 1,850 of 48, 1,610 of 25).
namespace {
constexpr int kMaxPieces = 256;
constexpr int64_t kPieceChunks = 32;
constexpr int kMaxDevices = 64;
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t start = nullptr, done[kMaxPieces] = {};
    bool ok = false, tried = false;
};
SideStream g_side[kMaxDevices];
std::mutex g_side_mu;   // one call's fork and join are enqueued as a whole

// pieces for this problem (1 = one prep and one state pass, as usual)
int64_t chunk_pieces(const gdn2_problem* p)
{
    const int64_t nt = nchunks(p), nch = p->B * nvh(p);
    if (p->B != 1 || nt < 256) return 1;
    const int vs = gdn2::chunk_state_slice(nch, (int)p->dv, (int)p->dk, (int)io_size(p));
    if (nch * (p->dv / vs) > 128) return 1;   // the state pass would hold more than half of the CUs
    const int64_t k = (nt + kPieceChunks - 1) / kPieceChunks;
    return k > kMaxPieces ? kMaxPieces : k;
}

SideStream* side_stream(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    SideStream& x = g_side[dev];
    if (!x.tried) {
        x.tried = true;
        bool ok = hipStreamCreateWithFlags(&x.s, hipStreamNonBlocking) == hipSuccess;
        ok = ok && hipEventCreateWithFlags(&x.start, hipEventDisableTiming) == hipSuccess;
        for (int i = 0; i < kMaxPieces && ok; ++i)
            ok = hipEventCreateWithFlags(&x.done[i], hipEventDisableTiming) == hipSuccess;
        x.ok = ok;
    }
    return x.ok ? &x : nullptr;
}

// the forward in npc pieces (B == 1): pointers of piece i are offset by its
// first token; its workspace blocks follow the previous pieces'
int chunk_fwd_pieces(const gdn2_problem* p, int64_t npc, const void* q, const void* k, const void* v,
                     const void* alpha, const void* b, const void* w, const float* S0, void* o, float* S_out,
                     void* workspace, hipStream_t s)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GDN2_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream* side = side_stream(dev);
    if (side == nullptr) return GDN2_ERR_DEVICE;
    const int64_t nt = nchunks(p), per = (nt + npc - 1) / npc;
    const int64_t es = io_size(p), gs = gates_bf16(p) ? 2 : 4, Hv = nvh(p);
    const int64_t blk = ws_block_bytes(p);
    auto piece = [&](int64_t i, gdn2_problem* pp, int64_t* t0, int64_t* wsoff) {
        const int64_t c0 = i * per, c1 = (i + 1) * per < nt ? (i + 1) * per : nt;
        *pp = *p;
        *t0 = c0 * 64;
        pp->T = (c1 * 64 < p->T ? c1 * 64 : p->T) - *t0;
        *wsoff = c0 * Hv * blk;   // blocks of the pieces before, B == 1
    };
    auto at = [](const void* x, int64_t bytes) { return static_cast<const char*>(x) + bytes; };
    // the side stream starts after everything already on the caller's stream
    if (hipEventRecord(side->start, s) != hipSuccess || hipStreamWaitEvent(side->s, side->start, 0) != hipSuccess)
        return GDN2_ERR_DEVICE;
    for (int64_t i = 0; i < npc; ++i) {
        gdn2_problem pp;
        int64_t t0, wso;
        piece(i, &pp, &t0, &wso);
        if (pp.T <= 0) break;
        const int64_t tk = t0 * p->H * p->dk, tg = t0 * Hv * p->dk, tv = t0 * Hv * p->dv;
        const hipStream_t ps = i == 0 ? s : side->s;
        int st = do_prep(&pp, at(q, tk * es), at(k, tk * es), at(v, tv * es), at(alpha, tg * gs), at(b, tg * gs),
                         at(w, tv * gs), static_cast<char*>(workspace) + wso, ps);
        if (st) return st;
        if (i > 0 && hipEventRecord(side->done[i], side->s) != hipSuccess) return GDN2_ERR_DEVICE;
    }
    for (int64_t i = 0; i < npc; ++i) {
        gdn2_problem pp;
        int64_t t0, wso;
        piece(i, &pp, &t0, &wso);
        if (pp.T <= 0) break;
        if (i > 0 && hipStreamWaitEvent(s, side->done[i], 0) != hipSuccess) return GDN2_ERR_DEVICE;
        const int64_t tv = t0 * Hv * p->dv;
        int st = do_state(&pp, i == 0 ? S0 : S_out, static_cast<char*>(o) + tv * es, S_out,
                          static_cast<char*>(workspace) + wso, s);
        if (st) return st;
    }
    return GDN2_OK;
}
}  // namespace

int gdn2_chunk_fwd(const gdn2_problem* p, const void* q, const void* k, const void* v,
                   const void* alpha, const void* b, const void* w, const float* S0, void* o,
                   float* S_out, void* workspace, size_t workspace_bytes, void* stream)
{
    int st = check_problem(p, true);
    if (st) return st;
    st = check_inputs(p, q, k, v, alpha, b, w, o);
    if (st) return st;
    const int64_t need = fwd_ws_bytes(p);
    if (need > 0 && (workspace == nullptr || static_cast<int64_t>(workspace_bytes) < need))
        return GDN2_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_WORKSPACE;
    const Sizes z = sizes_of(p);
    const Range ins[7] = {range_of(q, z.key),  range_of(k, z.key),  range_of(v, z.val),
                          range_of(alpha, z.gk), range_of(b, z.gk), range_of(w, z.gv),
                          range_of(S0, z.state)};
    const Range outs[3] = {range_of(o, z.val), range_of(S_out, z.state), range_of(workspace, need)};
    st = check_alias(outs, 3, ins, 7, S0, S_out, 6, 1);
    if (st) return st;
    st = check_align({q, k, v, alpha, b, w, S0, o, S_out});
    if (st) return st;
    if (p->B * p->H == 0 || (nchunks(p) == 0 && S_out == S0)) return GDN2_OK;
    st = device_ready();
    if (st) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // pieces only outside stream capture (no stream is created or forked then)
    const int64_t npc = chunk_pieces(p);
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (npc > 1 && S_out != nullptr && hipStreamIsCapturing(s, &cap) == hipSuccess && cap == hipStreamCaptureStatusNone)
        return chunk_fwd_pieces(p, npc, q, k, v, alpha, b, w, S0, o, S_out, workspace, s);
    st = do_prep(p, q, k, v, alpha, b, w, workspace, s);
    if (st) return st;
    return do_state(p, S0, o, S_out, workspace, s);
}

int gdn2_chunk_fwd_noalloc(const gdn2_problem* p, const void* q, const void* k, const void* v,
                           const void* alpha, const void* b, const void* w, const float* S0, void* o,
                           float* S_out, void* stream)
{
    int st = check_problem(p, true);
    if (st) return st;
    st = check_inputs(p, q, k, v, alpha, b, w, o);
    if (st) return st;
    const int64_t need = fwd_ws_bytes(p);
    if (need > static_cast<int64_t>(GDN2_NOALLOC_SCRATCH_BYTES)) return GDN2_ERR_WORKSPACE;
    const Sizes z = sizes_of(p);
    const Range ins[7] = {range_of(q, z.key),  range_of(k, z.key),  range_of(v, z.val),
                          range_of(alpha, z.gk), range_of(b, z.gk), range_of(w, z.gv),
                          range_of(S0, z.state)};
    const Range outs[2] = {range_of(o, z.val), range_of(S_out, z.state)};
    st = check_alias(outs, 2, ins, 7, S0, S_out, 6, 1);
    if (st) return st;
    st = check_align({q, k, v, alpha, b, w, S0, o, S_out});
    if (st) return st;
    if (p->B * p->H == 0 || (nchunks(p) == 0 && S_out == S0)) return GDN2_OK;
    st = device_ready();
    if (st) return st;
    // the device address of this GPU's copy of the library's scratch array
    const hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = need > 0 ? gdn2::noalloc_scratch() : nullptr;
    if (need > 0 && ws == nullptr) return GDN2_ERR_DEVICE;
    st = do_prep(p, q, k, v, alpha, b, w, ws, s);
    if (st) return st;
    return do_state(p, S0, o, S_out, ws, s);
}

int gdn2_chunk_fwd_conv(const gdn2_problem* p, const gdn2_conv* conv, const void* q, const void* k,
                        const void* v, const void* alpha, const void* b, const void* w, const float* S0,
                        void* o, float* S_out, void* workspace, size_t workspace_bytes, void* stream)
{
    int st = check_problem(p, true);
    if (st) return st;
    st = check_conv(p, conv);
    if (st) return st;
    st = check_inputs(p, q, k, v, alpha, b, w, o);
    if (st) return st;
    const int64_t need = fwd_ws_bytes(p);
    if (need > 0 && (workspace == nullptr || static_cast<int64_t>(workspace_bytes) < need))
        return GDN2_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_WORKSPACE;
    const Sizes z = sizes_of(p);
    const Range cin = conv_state_range(p, conv, conv->state_in), cout = conv_state_range(p, conv, conv->state_out);
    const Range ins[9] = {range_of(q, z.key),  range_of(k, z.key),  range_of(v, z.val),
                          range_of(alpha, z.gk), range_of(b, z.gk), range_of(w, z.gv),
                          range_of(S0, z.state), conv_weight_range(p, conv), cin};
    const Range outs[4] = {range_of(o, z.val), range_of(S_out, z.state), range_of(workspace, need), cout};
    // the window may be updated in place (equal pointers), like the state
    st = check_alias(outs, 3, ins, 9, S0, S_out, 6, 1);
    if (st) return st;
    for (int j = 0; j < 8; ++j)
        if (overlap(cout, ins[j])) return GDN2_ERR_ALIAS;
    if (overlap(cout, cin) && conv->state_out != conv->state_in) return GDN2_ERR_ALIAS;
    for (int j = 0; j < 3; ++j)
        if (overlap(cout, outs[j])) return GDN2_ERR_ALIAS;
    st = check_align({q, k, v, alpha, b, w, S0, o, S_out, conv->weight, conv->state_in, conv->state_out});
    if (st) return st;
    if (p->B * p->H == 0 || (nchunks(p) == 0 && S_out == S0 && !conv_window_moves(conv))) return GDN2_OK;
    st = device_ready();
    if (st) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = do_prep(p, q, k, v, alpha, b, w, workspace, s, conv);
    if (st) return st;
    return do_state(p, S0, o, S_out, workspace, s, conv, q, k, v);
}

int gdn2_recurrent_step(const gdn2_problem* p, const void* q, const void* k, const void* v,
                        const void* alpha, const void* b, const void* w, const float* S_in, void* o,
                        float* S_out, void* stream)
{
    int st = check_problem(p, false);
    if (st) return st;
    st = check_inputs(p, q, k, v, alpha, b, w, o);
    if (st) return st;
    const Sizes z = sizes_of(p);
    const Range ins[7] = {range_of(q, z.key),  range_of(k, z.key),  range_of(v, z.val),
                          range_of(alpha, z.gk), range_of(b, z.gk), range_of(w, z.gv),
                          range_of(S_in, z.state)};
    const Range outs[2] = {range_of(o, z.val), range_of(S_out, z.state)};
    st = check_alias(outs, 2, ins, 7, S_in, S_out, 6, 1);
    if (st) return st;
    st = check_align({q, k, v, alpha, b, w, S_in, o, S_out});
    if (st) return st;
    const int64_t nch = p->B * nvh(p);
    if (nch == 0) return GDN2_OK;
    if (p->T == 0 && S_out == S_in) return GDN2_OK;
    st = device_ready();
    if (st) return st;
    const int vs = gdn2::recurrent_slice(nch, p->T, (int)p->dv);
    gdn2::RecArgs a{q, k, v, alpha, b, w, S_in, o, S_out, p->B, p->T, nvh(p), p->H, (int)p->dv,
                    (int)(p->dv / vs), (int)p->flags, nullptr};
    return launch_status(gdn2::launch_recurrent(a, (int)p->dk, vs, is_bf16(p), gates_bf16(p),
                                                static_cast<hipStream_t>(stream)));
}

int gdn2_recurrent_step_conv(const gdn2_problem* p, const gdn2_conv* conv, const void* q, const void* k,
                             const void* v, const void* alpha, const void* b, const void* w,
                             const float* S_in, void* o, float* S_out, void* stream)
{
    int st = check_problem(p, false);
    if (st) return st;
    st = check_conv(p, conv);
    if (st) return st;
    st = check_inputs(p, q, k, v, alpha, b, w, o);
    if (st) return st;
    const Sizes z = sizes_of(p);
    const Range cout = conv_state_range(p, conv, conv->state_out);
    const Range ins[9] = {range_of(q, z.key),  range_of(k, z.key),  range_of(v, z.val),
                          range_of(alpha, z.gk), range_of(b, z.gk), range_of(w, z.gv),
                          range_of(S_in, z.state), conv_weight_range(p, conv),
                          conv_state_range(p, conv, conv->state_in)};
    const Range outs[3] = {range_of(o, z.val), range_of(S_out, z.state), cout};
    // the state may be updated in place; the window not (workgroups of one
    // sequence read it while the first of them writes)
    st = check_alias(outs, 3, ins, 9, S_in, S_out, 6, 1);
    if (st) return st;
    st = check_align({q, k, v, alpha, b, w, S_in, o, S_out, conv->weight, conv->state_in, conv->state_out});
    if (st) return st;
    const int64_t nch = p->B * nvh(p);
    if (nch == 0) return GDN2_OK;
    if (p->T == 0 && S_out == S_in && !conv_window_moves(conv)) return GDN2_OK;
    st = device_ready();
    if (st) return st;
    const int vs = gdn2::recurrent_slice(nch, p->T, (int)p->dv);
    gdn2::RecArgs a{q, k, v, alpha, b, w, S_in, o, S_out, p->B, p->T, nvh(p), p->H, (int)p->dv,
                    (int)(p->dv / vs), (int)p->flags, nullptr};
    a.conv_w = conv->weight;
    a.conv_in = conv->K > 1 ? conv->state_in : nullptr;
    a.conv_out = conv->K > 1 ? conv->state_out : nullptr;
    a.conv_C = conv_channels(p);
    a.conv_K = conv->K;
    a.conv_silu = (conv->flags & GDN2_CONV_SILU) != 0;
    return launch_status(gdn2::launch_recurrent(a, (int)p->dk, vs, is_bf16(p), gates_bf16(p),
                                                static_cast<hipStream_t>(stream)));
}

int gdn2_recurrent_step_gated(const gdn2_problem* p, const void* q, const void* k, const void* v,
                              const void* alpha, const void* b, const void* w, const float* S_in,
                              const void* g, const float* norm_weight, void* y, float* S_out, void* stream)
{
    int st = check_problem(p, false);
    if (st) return st;
    // whole rows in one workgroup: dv one of the widths the kernel is built for
    if (p->dv != 16 && p->dv != 32 && p->dv != 64 && p->dv != 128 && p->dv != 256) return GDN2_ERR_SHAPE;
    st = check_inputs(p, q, k, v, alpha, b, w, y);
    if (st) return st;
    if (rows_nonempty(p) && (g == nullptr || norm_weight == nullptr)) return GDN2_ERR_NULL;
    const Sizes z = sizes_of(p);
    const Range ins[9] = {range_of(q, z.key),  range_of(k, z.key),  range_of(v, z.val),
                          range_of(alpha, z.gk), range_of(b, z.gk), range_of(w, z.gv),
                          range_of(S_in, z.state), range_of(g, z.val), range_of(norm_weight, p->dv * 4)};
    const Range outs[2] = {range_of(y, z.val), range_of(S_out, z.state)};
    st = check_alias(outs, 2, ins, 9, S_in, S_out, 6, 1);
    if (st) return st;
    st = check_align({q, k, v, alpha, b, w, S_in, y, S_out, g, norm_weight});
    if (st) return st;
    const int64_t nch = p->B * nvh(p);
    if (nch == 0) return GDN2_OK;
    if (p->T == 0 && S_out == S_in) return GDN2_OK;
    st = device_ready();
    if (st) return st;
    // one workgroup holds whole value rows, so the row statistic is local
    gdn2::RecArgs a{q, k, v, alpha, b, w, S_in, y, S_out, p->B, p->T, nvh(p), p->H, (int)p->dv,
                    1, (int)p->flags, nullptr, g, norm_weight, 1e-5f};
    return launch_status(gdn2::launch_recurrent(a, (int)p->dk, (int)p->dv, is_bf16(p), gates_bf16(p),
                                                static_cast<hipStream_t>(stream)));
}

size_t gdn2_chunk_fwd_varlen_workspace_size(const gdn2_problem* p)
{
    if (check_problem(p, true, true) != GDN2_OK) return 0;
    return static_cast<size_t>(varlen_ws_bytes(p));
}

int gdn2_chunk_fwd_varlen(const gdn2_problem* p, const int32_t* cu_seqlens, const void* q, const void* k,
                          const void* v, const void* alpha, const void* b, const void* w, const float* S0,
                          void* o, float* S_out, void* workspace, size_t workspace_bytes, void* stream)
{
    int st = check_problem(p, true, true);
    if (st) return st;
    st = check_cu(p, cu_seqlens);
    if (st) return st;
    const bool any = p->B * nvh(p) > 0;
    if (any) {
        st = check_inputs(p, q, k, v, alpha, b, w, o);
        if (st) return st;
    }
    const int64_t need = any ? varlen_ws_bytes(p) : 0;
    if (need > 0 && (workspace == nullptr || static_cast<int64_t>(workspace_bytes) < need))
        return GDN2_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_WORKSPACE;
    const Sizes z = sizes_of(p, true);
    const Range ins[8] = {range_of(q, z.key),  range_of(k, z.key),  range_of(v, z.val),
                          range_of(alpha, z.gk), range_of(b, z.gk), range_of(w, z.gv),
                          range_of(S0, z.state), range_of(cu_seqlens, any ? 4 * (p->B + 1) : 0)};
    const Range outs[3] = {range_of(o, z.val), range_of(S_out, z.state), range_of(workspace, need)};
    st = check_alias(outs, 3, ins, 8, S0, S_out, 6, 1);
    if (st) return st;
    st = check_align({q, k, v, alpha, b, w, S0, o, S_out});
    if (st) return st;
    if (!any || (p->T == 0 && (S_out == S0 || S_out == nullptr))) return GDN2_OK;
    st = device_ready();
    if (st) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int* plan = static_cast<int*>(workspace);
    char* blocks = static_cast<char*>(workspace) + varlen_plan_bytes(p);
    const int64_t ncmax = varlen_ncmax(p);
    st = launch_status(gdn2::launch_varlen_plan(gdn2::PlanArgs{cu_seqlens, plan, p->B, p->T, ncmax}, s));
    if (st) return st;
    if (p->T > 0) {
        gdn2::PrepArgs a{q, k, v, alpha, b, w, blocks, ws_block_bytes(p), p->B, p->T, nvh(p), p->H,
                         (int)p->dv, 0, (int)p->flags, plan, ncmax};
        st = launch_status(gdn2::launch_chunk_prep(a, (int)p->dk, is_bf16(p), gates_bf16(p), s));
        if (st) return st;
    }
    const int64_t nch = p->B * nvh(p);
    const int vs = gdn2::chunk_state_slice(nch, (int)p->dv, (int)p->dk, (int)io_size(p));
    gdn2::StateArgs a{blocks, ws_block_bytes(p), S0, o, S_out, p->B, p->T, nvh(p), (int)p->dv, 0,
                      (int)(p->dv / vs), plan, ncmax};
    return launch_status(gdn2::launch_chunk_state(a, (int)p->dk, vs, is_bf16(p), s));
}

int gdn2_recurrent_varlen(const gdn2_problem* p, const int32_t* cu_seqlens, const void* q, const void* k,
                          const void* v, const void* alpha, const void* b, const void* w, const float* S_in,
                          void* o, float* S_out, void* stream)
{
    int st = check_problem(p, false, true);
    if (st) return st;
    st = check_cu(p, cu_seqlens);
    if (st) return st;
    const int64_t nch = p->B * nvh(p);
    if (nch > 0) {
        st = check_inputs(p, q, k, v, alpha, b, w, o);
        if (st) return st;
    }
    const Sizes z = sizes_of(p, true);
    const Range ins[8] = {range_of(q, z.key),  range_of(k, z.key),  range_of(v, z.val),
                          range_of(alpha, z.gk), range_of(b, z.gk), range_of(w, z.gv),
                          range_of(S_in, z.state), range_of(cu_seqlens, nch > 0 ? 4 * (p->B + 1) : 0)};
    const Range outs[2] = {range_of(o, z.val), range_of(S_out, z.state)};
    st = check_alias(outs, 2, ins, 8, S_in, S_out, 6, 1);
    if (st) return st;
    st = check_align({q, k, v, alpha, b, w, S_in, o, S_out});
    if (st) return st;
    if (nch == 0 || (p->T == 0 && (S_out == S_in || S_out == nullptr))) return GDN2_OK;
    st = device_ready();
    if (st) return st;
    // slice width from the mean sequence length
    const int vs = gdn2::recurrent_slice(nch, p->T / p->B, (int)p->dv);
    gdn2::RecArgs a{q, k, v, alpha, b, w, S_in, o, S_out, p->B, p->T, nvh(p), p->H, (int)p->dv,
                    (int)(p->dv / vs), (int)p->flags, cu_seqlens};
    return launch_status(gdn2::launch_recurrent(a, (int)p->dk, vs, is_bf16(p), gates_bf16(p),
                                                static_cast<hipStream_t>(stream)));
}

size_t gdn2_chunk_bwd_workspace_size(const gdn2_problem* p)
{
    if (check_problem(p, true) != GDN2_OK) return 0;
    return static_cast<size_t>(bwd_wrap(p).total);
}

int gdn2_chunk_bwd(const gdn2_problem* p, const void* q, const void* k, const void* v, const void* alpha,
                   const void* b, const void* w, const float* S0, const void* dO, const float* dS_T, void* dq,
                   void* dk, void* dv, void* dalpha, void* db, void* dw, float* dS0, void* workspace,
                   size_t workspace_bytes, void* stream)
{
    int st = check_problem(p, true);
    if (st) return st;
    st = check_inputs(p, q, k, v, alpha, b, w, dO);
    if (st) return st;
    if (rows_nonempty(p) && (!dq || !dk || !dv || !dalpha || !db || !dw)) return GDN2_ERR_NULL;
    const BwdWrap wr = bwd_wrap(p);
    const int64_t need = p->B * p->H > 0 ? wr.total : 0;
    if (need > 0 && (workspace == nullptr || static_cast<int64_t>(workspace_bytes) < need))
        return GDN2_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_WORKSPACE;
    const Sizes z = sizes_of(p);
    const Range ins[9] = {range_of(q, z.key),  range_of(k, z.key),  range_of(v, z.val),
                          range_of(alpha, z.gk), range_of(b, z.gk), range_of(w, z.gv),
                          range_of(S0, z.state), range_of(dO, z.val), range_of(dS_T, z.state)};
    const Range outs[8] = {range_of(dq, z.key),  range_of(dk, z.key), range_of(dv, z.val),
                           range_of(dalpha, z.gk), range_of(db, z.gk), range_of(dw, z.gv),
                           range_of(dS0, z.state), range_of(workspace, need)};
    st = check_alias(outs, 8, ins, 9, nullptr, nullptr, -1, -1);
    if (st) return st;
    st = check_align({q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk, dv, dalpha, db, dw, dS0});
    if (st) return st;
    if (p->B * p->H == 0) return GDN2_OK;
    if (nchunks(p) == 0 && dS0 == nullptr) return GDN2_OK;
    st = device_ready();
    if (st) return st;
    return bwd_run(p, wr, nullptr, q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk, dv, dalpha, db, dw, dS0,
                   static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

int gdn2_gated_rmsnorm(const gdn2_problem* p, const void* o, const void* g, const float* weight, void* y,
                       void* stream)
{
    int st = check_problem(p, false);
    if (st) return st;
    const int64_t rows = p->B * p->T * nvh(p);
    if (rows == 0) return GDN2_OK;
    if (!o || !g || !weight || !y) return GDN2_ERR_NULL;
    const Sizes z = sizes_of(p);
    const Range ins[3] = {range_of(o, z.val), range_of(g, z.val), range_of(weight, p->dv * 4)};
    const Range outs[1] = {range_of(y, z.val)};
    st = check_alias(outs, 1, ins, 3, o, y, 0, 0);
    if (st) return st;
    st = check_align({o, g, weight, y});
    if (st) return st;
    st = device_ready();
    if (st) return st;
    gdn2::NormArgs a{o, g, weight, y, rows, (int)p->dv, 1.0f / (float)p->dv, 1e-5f};
    return launch_status(gdn2::launch_gated_rmsnorm(a, is_bf16(p), static_cast<hipStream_t>(stream)));
}

// sizes of the short convolution; a non-zero return is the status
static int conv_check(int64_t B, int64_t T, int64_t C, int32_t K, int32_t flags, int32_t io_dtype)
{
    if (B < 0 || T < 0 || C <= 0 || B > kMaxDim || T > kMaxDim || C > kMaxDim) return GDN2_ERR_SHAPE;
    if (C % 8 != 0 || K < 1 || K > 8 || (flags & ~GDN2_CONV_SILU) != 0) return GDN2_ERR_SHAPE;
    // every element count and the forward's thread count must fit in 32 bits of workgroups
    const double n = (double)B * (double)T * (double)C;
    if (n > 1e15 || n / (32.0 * 256.0) > 2.0e9) return GDN2_ERR_SHAPE;
    if (io_dtype != GDN2_F32 && io_dtype != GDN2_BF16) return GDN2_ERR_DTYPE;
    return GDN2_OK;
}

static int64_t conv_spans(int64_t T) { return T == 0 ? 1 : (T + gdn2::kConvSpan - 1) / gdn2::kConvSpan; }

int gdn2_short_conv(int64_t B, int64_t T, int64_t C, int32_t K, int32_t flags, int32_t io_dtype,
                    const void* x, const float* weight, const void* state_in,
                    void* y, void* state_out, void* stream)
{
    int st = conv_check(B, T, C, K, flags, io_dtype);
    if (st) return st;
    if (K == 1) state_in = state_out = nullptr;
    const int64_t es = io_dtype == GDN2_BF16 ? 2 : 4;
    const int64_t span = gdn2::kConvSpanF(io_dtype == GDN2_BF16);
    int64_t ntile = (T + span - 1) / span;
    if (ntile == 0 && state_out != nullptr) ntile = 1;
    if (B == 0 || ntile == 0) return GDN2_OK;
    if (!weight) return GDN2_ERR_NULL;
    if (T > 0 && (!x || !y)) return GDN2_ERR_NULL;
    const int64_t xb = B * T * C * es, sb = B * (K - 1) * C * es;
    const Range ins[3] = {range_of(x, xb), range_of(weight, C * K * 4), range_of(state_in, sb)};
    const Range outs[2] = {range_of(y, xb), range_of(state_out, sb)};
    st = check_alias(outs, 2, ins, 3, state_in, state_out, 2, 1);
    if (st) return st;
    st = check_align({x, weight, state_in, y, state_out});
    if (st) return st;
    st = device_ready();
    if (st) return st;
    gdn2::ConvArgs a{x, weight, state_in, y, state_out, B, T, C, ntile};
    return launch_status(gdn2::launch_short_conv(a, K, (flags & GDN2_CONV_SILU) != 0, io_dtype == GDN2_BF16,
                                                 static_cast<hipStream_t>(stream)));
}

size_t gdn2_short_conv_bwd_workspace_size(int64_t B, int64_t T, int64_t C, int32_t K)
{
    if (conv_check(B, T, C, K, 0, GDN2_F32) != GDN2_OK) return 0;
    return (size_t)(B * conv_spans(T) * C * K) * sizeof(float);
}

int gdn2_short_conv_bwd(int64_t B, int64_t T, int64_t C, int32_t K, int32_t flags, int32_t io_dtype,
                        const void* x, const float* weight, const void* state_in, const void* dy,
                        const void* dstate_out, void* dx, float* dweight, void* dstate_in,
                        void* workspace, size_t workspace_bytes, void* stream)
{
    int st = conv_check(B, T, C, K, flags, io_dtype);
    if (st) return st;
    if (K == 1) {
        state_in = dstate_out = nullptr;
        dstate_in = nullptr;
    }
    if (!weight || !dweight) return GDN2_ERR_NULL;
    if (B > 0 && T > 0 && (!x || !dy || !dx)) return GDN2_ERR_NULL;
    const size_t need = gdn2_short_conv_bwd_workspace_size(B, T, C, K);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GDN2_ERR_WORKSPACE;
    const int64_t es = io_dtype == GDN2_BF16 ? 2 : 4;
    const int64_t xb = B * T * C * es, sb = B * (K - 1) * C * es;
    const Range ins[5] = {range_of(x, xb), range_of(weight, C * K * 4), range_of(state_in, sb), range_of(dy, xb),
                          range_of(dstate_out, sb)};
    const Range outs[4] = {range_of(dx, xb), range_of(dweight, C * K * 4), range_of(dstate_in, sb),
                           range_of(workspace, (int64_t)need)};
    st = check_alias(outs, 4, ins, 5, nullptr, nullptr, -1, -1);
    if (st) return st;
    st = check_align({x, weight, state_in, dy, dstate_out, dx, dweight, dstate_in, workspace});
    if (st) return st;
    st = device_ready();
    if (st) return st;
    gdn2::ConvBwdArgs a{x, weight, state_in, dy, dx, dweight, dstate_in, static_cast<float*>(workspace),
                        dstate_out, B, T, C, conv_spans(T)};
    return launch_status(gdn2::launch_short_conv_bwd(a, K, (flags & GDN2_CONV_SILU) != 0, io_dtype == GDN2_BF16,
                                                     static_cast<hipStream_t>(stream)));
}

size_t gdn2_chunk_bwd_varlen_workspace_size(const gdn2_problem* p)
{
    if (check_problem(p, true, true) != GDN2_OK) return 0;
    if (p->B * nvh(p) == 0) return 0;
    return static_cast<size_t>(bwd_wrap(p, true).total);
}

int gdn2_chunk_bwd_varlen(const gdn2_problem* p, const int32_t* cu_seqlens, const void* q, const void* k,
                          const void* v, const void* alpha, const void* b, const void* w, const float* S0,
                          const void* dO, const float* dS_T, void* dq, void* dk, void* dv, void* dalpha, void* db,
                          void* dw, float* dS0, void* workspace, size_t workspace_bytes, void* stream)
{
    int st = check_problem(p, true, true);
    if (st) return st;
    st = check_cu(p, cu_seqlens);
    if (st) return st;
    const bool any = p->B * nvh(p) > 0;
    if (any) {
        st = check_inputs(p, q, k, v, alpha, b, w, dO);
        if (st) return st;
        if (rows_nonempty(p) && (!dq || !dk || !dv || !dalpha || !db || !dw)) return GDN2_ERR_NULL;
    }
    const BwdWrap wr = bwd_wrap(p, true);
    const int64_t need = any ? wr.total : 0;
    if (need > 0 && (workspace == nullptr || static_cast<int64_t>(workspace_bytes) < need))
        return GDN2_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_WORKSPACE;
    const Sizes z = sizes_of(p, true);
    const Range ins[10] = {range_of(q, z.key),   range_of(k, z.key),  range_of(v, z.val),
                           range_of(alpha, z.gk), range_of(b, z.gk),   range_of(w, z.gv),
                           range_of(S0, z.state), range_of(dO, z.val), range_of(dS_T, z.state),
                           range_of(cu_seqlens, any ? 4 * (p->B + 1) : 0)};
    const Range outs[8] = {range_of(dq, z.key),   range_of(dk, z.key), range_of(dv, z.val),
                           range_of(dalpha, z.gk), range_of(db, z.gk),  range_of(dw, z.gv),
                           range_of(dS0, z.state), range_of(workspace, need)};
    st = check_alias(outs, 8, ins, 10, nullptr, nullptr, -1, -1);
    if (st) return st;
    st = check_align({q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk, dv, dalpha, db, dw, dS0});
    if (st) return st;
    if (!any) return GDN2_OK;
    if (p->T == 0 && dS0 == nullptr) return GDN2_OK;
    st = device_ready();
    if (st) return st;
    return bwd_run(p, wr, cu_seqlens, q, k, v, alpha, b, w, S0, dO, dS_T, dq, dk, dv, dalpha, db, dw, dS0,
                   static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

}  // extern "C"
