// Host-only exercise of libgdn2's C-ABI layer, built with AddressSanitizer and
// UndefinedBehaviorSanitizer against the stand-ins in host_stubs.cpp.
//
// Every entry point is called once with valid arguments (it must return
// GDN2_OK and launch, every launch-argument check passing) and then with a
// set of broken arguments, each of which must return its documented code
// before anything is launched.  Workspace-size queries are also fed sizes at
// and past the documented limits.  Exit status 0 means every case held; the
// sanitizers abort the process on any memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gdn2.h"
#include "host_stubs.hpp"

namespace {

int g_bad = 0;

// a failing call launches nothing; a valid one launches [lo, hi] times
void expect(const char* what, int got, int want, int lo = 0, int hi = 0)
{
    const int n = stub::launches();
    const bool launch_rule = want == GDN2_OK ? (n >= lo && n <= hi) : n == 0;
    if (got != want || !launch_rule) {
        std::fprintf(stderr, "FAIL %s: status %d (want %d), %d launches\n", what, got, want, n);
        ++g_bad;
    }
    stub::reset_launches();
}

// one problem's device tensors
struct Tensors {
    gdn2_problem p;
    size_t esz, gsz;
    void *q, *k, *v, *alpha, *b, *w, *o, *g, *y;
    float *S0, *S_out, *norm_w;
    void* ws;
    size_t ws_bytes;
};

int64_t nvh(const gdn2_problem& p) { return p.Hv ? p.Hv : p.H; }

Tensors make(int64_t B, int64_t T, int64_t H, int64_t Hv, int64_t dk, int64_t dv, int io, int gate, int flags)
{
    Tensors t{};
    t.p = gdn2_problem{B, T, H, dk, dv, 64, io, gate, flags, Hv};
    t.esz = io == GDN2_BF16 ? 2 : 4;
    t.gsz = gate == GDN2_BF16 ? 2 : 4;
    const int64_t tok = B * T, hv = nvh(t.p);
    t.q = stub::dev_alloc(tok * H * dk * t.esz);
    t.k = stub::dev_alloc(tok * H * dk * t.esz);
    t.v = stub::dev_alloc(tok * hv * dv * t.esz);
    t.o = stub::dev_alloc(tok * hv * dv * t.esz);
    t.g = stub::dev_alloc(tok * hv * dv * t.esz);
    t.y = stub::dev_alloc(tok * hv * dv * t.esz);
    t.alpha = stub::dev_alloc(tok * hv * dk * t.gsz);
    t.b = stub::dev_alloc(tok * hv * dk * t.gsz);
    t.w = stub::dev_alloc(tok * hv * dv * t.gsz);
    t.S0 = static_cast<float*>(stub::dev_alloc(B * hv * dk * dv * 4));
    t.S_out = static_cast<float*>(stub::dev_alloc(B * hv * dk * dv * 4));
    t.norm_w = static_cast<float*>(stub::dev_alloc(dv * 4));
    t.ws_bytes = gdn2_chunk_fwd_workspace_size(&t.p);
    t.ws = stub::dev_alloc(t.ws_bytes);
    return t;
}

int fwd(const Tensors& t, const gdn2_problem* p, const void* q, void* o, const float* S0, float* S_out, void* ws,
        size_t wsb)
{
    return gdn2_chunk_fwd(p, q, t.k, t.v, t.alpha, t.b, t.w, S0, o, S_out, ws, wsb, nullptr);
}

void chunk_forward_cases()
{
    // a long single sequence with few chains: run in pieces (prep of the next
    // piece beside the state pass); every piece's pointers must stay inside
    // the tensors and its workspace blocks inside the workspace
    for (int io = 0; io < 2; ++io) {
        Tensors t = make(1, 256 * 64 + 37, 2, 4, 16, 16, io, io ? GDN2_BF16 : GDN2_F32, 0);
        const gdn2_problem& p = t.p;
        // 257 chunks: 9 pieces of at most 32 chunks, a prep and a state pass each
        expect("fwd long sequence in pieces", fwd(t, &p, t.q, t.o, t.S0, t.S_out, t.ws, t.ws_bytes), GDN2_OK, 18, 18);
        expect("fwd long sequence in pieces, in place", fwd(t, &p, t.q, t.o, t.S0, t.S0, t.ws, t.ws_bytes), GDN2_OK,
               18, 18);
        expect("fwd long sequence, no final state", fwd(t, &p, t.q, t.o, t.S0, nullptr, t.ws, t.ws_bytes), GDN2_OK,
               2, 2);
    }
    for (int io = 0; io < 2; ++io) {
        Tensors t = make(2, 100, 2, 4, 64, 32, io, GDN2_F32, io ? GDN2_FLAG_GATE_LOGITS | GDN2_FLAG_QK_L2NORM : 0);
        const gdn2_problem& p = t.p;
        expect("fwd valid", fwd(t, &p, t.q, t.o, t.S0, t.S_out, t.ws, t.ws_bytes), GDN2_OK, 2, 2);
        expect("fwd in-place state", fwd(t, &p, t.q, t.o, t.S0, t.S0, t.ws, t.ws_bytes), GDN2_OK, 2, 2);
        expect("fwd no states", fwd(t, &p, t.q, t.o, nullptr, nullptr, t.ws, t.ws_bytes), GDN2_OK, 2, 2);
        expect("prep valid", gdn2_chunk_prep(&p, t.q, t.k, t.v, t.alpha, t.b, t.w, t.ws, t.ws_bytes, nullptr),
               GDN2_OK, 1, 1);
        expect("state valid", gdn2_chunk_state(&p, t.S0, t.o, t.S_out, t.ws, t.ws_bytes, nullptr), GDN2_OK, 1, 1);
        expect("noalloc valid",
               gdn2_chunk_fwd_noalloc(&p, t.q, t.k, t.v, t.alpha, t.b, t.w, t.S0, t.o, t.S_out, nullptr), GDN2_OK, 2, 2);

        expect("fwd null problem", fwd(t, nullptr, t.q, t.o, t.S0, t.S_out, t.ws, t.ws_bytes), GDN2_ERR_NULL);
        expect("fwd null q", fwd(t, &p, nullptr, t.o, t.S0, t.S_out, t.ws, t.ws_bytes), GDN2_ERR_NULL);
        expect("fwd null o", fwd(t, &p, t.q, nullptr, t.S0, t.S_out, t.ws, t.ws_bytes), GDN2_ERR_NULL);
        expect("fwd misaligned q", fwd(t, &p, static_cast<const char*>(t.q) + 2, t.o, t.S0, t.S_out, t.ws, t.ws_bytes),
               GDN2_ERR_ALIGN);
        expect("fwd o over q", fwd(t, &p, t.q, t.q, t.S0, t.S_out, t.ws, t.ws_bytes), GDN2_ERR_ALIAS);
        expect("fwd S_out over S0 (shifted)", fwd(t, &p, t.q, t.o, t.S0, t.S0 + 4, t.ws, t.ws_bytes), GDN2_ERR_ALIAS);
        expect("fwd workspace over o", fwd(t, &p, t.q, t.o, t.S0, t.S_out, t.o, t.ws_bytes), GDN2_ERR_ALIAS);
        expect("fwd workspace short", fwd(t, &p, t.q, t.o, t.S0, t.S_out, t.ws, t.ws_bytes - 1), GDN2_ERR_WORKSPACE);
        expect("fwd workspace null", fwd(t, &p, t.q, t.o, t.S0, t.S_out, nullptr, t.ws_bytes), GDN2_ERR_WORKSPACE);
        expect("fwd workspace misaligned", fwd(t, &p, t.q, t.o, t.S0, t.S_out, static_cast<char*>(t.ws) + 16,
                                               t.ws_bytes), GDN2_ERR_WORKSPACE);
        struct {
            const char* what;
            void (*edit)(gdn2_problem&);
            int want;
        } shapes[] = {
            {"dk 48", [](gdn2_problem& q) { q.dk = 48; }, GDN2_ERR_SHAPE},
            {"dv 8", [](gdn2_problem& q) { q.dv = 8; }, GDN2_ERR_SHAPE},
            {"dv 264", [](gdn2_problem& q) { q.dv = 264; }, GDN2_ERR_SHAPE},
            {"chunk 32", [](gdn2_problem& q) { q.chunk = 32; }, GDN2_ERR_SHAPE},
            {"Hv 3", [](gdn2_problem& q) { q.Hv = 3; }, GDN2_ERR_SHAPE},
            {"flag 8", [](gdn2_problem& q) { q.flags = 8; }, GDN2_ERR_SHAPE},
            {"neg eigval alone", [](gdn2_problem& q) { q.flags = GDN2_FLAG_NEG_EIGVAL; }, GDN2_ERR_SHAPE},
            {"B -1", [](gdn2_problem& q) { q.B = -1; }, GDN2_ERR_SHAPE},
            {"T 2^41", [](gdn2_problem& q) { q.T = int64_t(1) << 41; }, GDN2_ERR_SHAPE},
            {"T 2^40 (too many rows)", [](gdn2_problem& q) { q.T = int64_t(1) << 40; }, GDN2_ERR_SHAPE},
            {"H int64 max", [](gdn2_problem& q) { q.H = INT64_MAX; }, GDN2_ERR_SHAPE},
            {"io dtype 7", [](gdn2_problem& q) { q.io_dtype = 7; }, GDN2_ERR_DTYPE},
            {"bf16 gates, fp32 io", [](gdn2_problem& q) { q.io_dtype = GDN2_F32; q.gate_dtype = GDN2_BF16; },
             GDN2_ERR_DTYPE},
        };
        for (auto& s : shapes) {
            gdn2_problem bad = p;
            s.edit(bad);
            expect(s.what, fwd(t, &bad, t.q, t.o, t.S0, t.S_out, t.ws, t.ws_bytes), s.want);
            if (s.want != GDN2_OK && gdn2_chunk_fwd_workspace_size(&bad) != 0) {
                std::fprintf(stderr, "FAIL %s: workspace size of an invalid problem\n", s.what);
                ++g_bad;
            }
        }
        // empty problems: nothing to compute; T = 0 still copies S0 into S_out
        gdn2_problem e = p;
        e.B = 0;
        expect("fwd B 0", fwd(t, &e, t.q, t.o, t.S0, t.S_out, t.ws, 0), GDN2_OK, 0, 0);
        e = p;
        e.T = 0;
        expect("fwd T 0 copies the state", fwd(t, &e, nullptr, nullptr, t.S0, t.S_out, nullptr, 0), GDN2_OK, 1, 1);
        expect("fwd T 0 in place", fwd(t, &e, nullptr, nullptr, t.S0, t.S0, nullptr, 0), GDN2_OK, 0, 0);
        // the library's fixed workspace is too small for this one
        gdn2_problem big = p;
        big.B = 1, big.T = 8192, big.H = 16, big.Hv = 0, big.dk = 128, big.dv = 128;
        Tensors tb = make(1, 8192, 16, 0, 128, 128, io, GDN2_F32, 0);
        expect("noalloc too large",
               gdn2_chunk_fwd_noalloc(&big, tb.q, tb.k, tb.v, tb.alpha, tb.b, tb.w, nullptr, tb.o, nullptr, nullptr),
               GDN2_ERR_WORKSPACE);
    }
}

void recurrent_cases()
{
    Tensors t = make(3, 5, 2, 2, 128, 64, GDN2_BF16, GDN2_BF16, 0);
    const gdn2_problem& p = t.p;
    auto rec = [&](const float* Sin, void* o, float* Sout) {
        return gdn2_recurrent_step(&p, t.q, t.k, t.v, t.alpha, t.b, t.w, Sin, o, Sout, nullptr);
    };
    expect("recurrent valid", rec(t.S0, t.o, t.S_out), GDN2_OK, 1, 1);
    expect("recurrent in place", rec(t.S0, t.o, t.S0), GDN2_OK, 1, 1);
    expect("recurrent o over S_in", rec(t.S0, t.S0, t.S_out), GDN2_ERR_ALIAS);
    expect("recurrent S_out over v", rec(t.S0, t.o, static_cast<float*>(t.v)), GDN2_ERR_ALIAS);
    auto gated = [&](const gdn2_problem* pp, const void* g, const float* nw, void* y) {
        return gdn2_recurrent_step_gated(pp, t.q, t.k, t.v, t.alpha, t.b, t.w, t.S0, g, nw, y, t.S_out, nullptr);
    };
    expect("gated valid", gated(&p, t.g, t.norm_w, t.y), GDN2_OK, 1, 1);
    expect("gated null g", gated(&p, nullptr, t.norm_w, t.y), GDN2_ERR_NULL);
    expect("gated null weight", gated(&p, t.g, nullptr, t.y), GDN2_ERR_NULL);
    expect("gated y over g", gated(&p, t.g, t.norm_w, t.g), GDN2_ERR_ALIAS);
    gdn2_problem odd = p;
    odd.dv = 48;
    expect("gated dv 48", gated(&odd, t.g, t.norm_w, t.y), GDN2_ERR_SHAPE);
    expect("rmsnorm valid", gdn2_gated_rmsnorm(&p, t.o, t.g, t.norm_w, t.y, nullptr), GDN2_OK, 1, 1);
    expect("rmsnorm in place", gdn2_gated_rmsnorm(&p, t.o, t.g, t.norm_w, t.o, nullptr), GDN2_OK, 1, 1);
    expect("rmsnorm y shifted over o",
           gdn2_gated_rmsnorm(&p, t.o, t.g, t.norm_w, static_cast<char*>(t.o) + 16, nullptr), GDN2_ERR_ALIAS);
}

void fused_conv_cases()
{
    for (int K : {1, 4}) {
        Tensors t = make(2, 100, 2, 4, 64, 32, GDN2_BF16, GDN2_F32, GDN2_FLAG_QK_L2NORM);
        const gdn2_problem& p = t.p;
        const int64_t C = 2 * 2 * 64 + 4 * 32;
        float* wt = static_cast<float*>(stub::dev_alloc(C * K * 4));
        void* sin = stub::dev_alloc(2 * 3 * C * 2);
        void* sout = stub::dev_alloc(2 * 3 * C * 2);
        gdn2_conv c{wt, sin, sout, K, GDN2_CONV_SILU};
        auto cf = [&](const gdn2_conv* cc, void* o) {
            return gdn2_chunk_fwd_conv(&p, cc, t.q, t.k, t.v, t.alpha, t.b, t.w, t.S0, o, t.S_out, t.ws, t.ws_bytes,
                                       nullptr);
        };
        auto rf = [&](const gdn2_conv* cc) {
            return gdn2_recurrent_step_conv(&p, cc, t.q, t.k, t.v, t.alpha, t.b, t.w, t.S0, t.o, t.S_out, nullptr);
        };
        expect("chunk conv valid", cf(&c, t.o), GDN2_OK, 2, 2);
        expect("recurrent conv valid", rf(&c), GDN2_OK, 1, 1);
        gdn2_conv inplace = c;
        inplace.state_out = sin;
        expect("chunk conv window in place", cf(&inplace, t.o), GDN2_OK, 2, 2);
        expect("recurrent conv window in place", rf(&inplace), K > 1 ? GDN2_ERR_ALIAS : GDN2_OK, 1, 1);
        expect("chunk conv null descriptor", cf(nullptr, t.o), GDN2_ERR_NULL);
        gdn2_conv bad = c;
        bad.weight = nullptr;
        expect("chunk conv null weight", cf(&bad, t.o), GDN2_ERR_NULL);
        bad = c;
        bad.K = 5;
        expect("conv K 5", rf(&bad), GDN2_ERR_SHAPE);
        bad = c;
        bad.flags = 2;
        expect("conv flag 2", cf(&bad, t.o), GDN2_ERR_SHAPE);
        bad = c;
        bad.state_out = t.q;
        if (K > 1) expect("conv window over q", cf(&bad, t.o), GDN2_ERR_ALIAS);
        expect("chunk conv o over weight", cf(&c, wt), GDN2_ERR_ALIAS);
        // no tokens: the window and the state are only carried over
        gdn2_problem e = p;
        e.T = 0;
        expect("chunk conv T 0", gdn2_chunk_fwd_conv(&e, &c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, t.S0,
                                                     nullptr, t.S_out, nullptr, 0, nullptr), GDN2_OK, 1, 1);
    }
}

void varlen_cases()
{
    // four packed sequences, 300 tokens in all
    Tensors t = make(1, 300, 2, 4, 64, 64, GDN2_BF16, GDN2_F32, 0);
    gdn2_problem p = t.p;
    p.B = 4;
    float* S0 = static_cast<float*>(stub::dev_alloc(4 * 4 * 64 * 64 * 4));
    float* Sout = static_cast<float*>(stub::dev_alloc(4 * 4 * 64 * 64 * 4));
    const int32_t* cu = static_cast<const int32_t*>(stub::dev_alloc(5 * 4));
    const size_t wsb = gdn2_chunk_fwd_varlen_workspace_size(&p);
    void* ws = stub::dev_alloc(wsb);
    auto cv = [&](const int32_t* c, void* w, size_t n) {
        return gdn2_chunk_fwd_varlen(&p, c, t.q, t.k, t.v, t.alpha, t.b, t.w, S0, t.o, Sout, w, n, nullptr);
    };
    expect("chunk varlen valid", cv(cu, ws, wsb), GDN2_OK, 3, 3);
    expect("chunk varlen null offsets", cv(nullptr, ws, wsb), GDN2_ERR_NULL);
    expect("chunk varlen misaligned offsets", cv(reinterpret_cast<const int32_t*>(
                                                   reinterpret_cast<const char*>(cu) + 2), ws, wsb),
           GDN2_ERR_ALIGN);
    expect("chunk varlen workspace short", cv(cu, ws, wsb - 256), GDN2_ERR_WORKSPACE);
    expect("recurrent varlen valid",
           gdn2_recurrent_varlen(&p, cu, t.q, t.k, t.v, t.alpha, t.b, t.w, S0, t.o, Sout, nullptr), GDN2_OK, 1, 1);
    expect("recurrent varlen o over offsets",
           gdn2_recurrent_varlen(&p, cu, t.q, t.k, t.v, t.alpha, t.b, t.w, S0, const_cast<int32_t*>(cu), Sout,
                                 nullptr),
           GDN2_ERR_ALIAS);
}

void backward_cases()
{
    // the matrix-core path (bf16, dk/dv in {32, 64, 128}) and the vector-ALU path
    const int64_t shapes[2][2] = {{64, 64}, {16, 48}};
    for (auto& s : shapes) {
        for (int flags : {0, GDN2_FLAG_GATE_LOGITS | GDN2_FLAG_NEG_EIGVAL | GDN2_FLAG_QK_L2NORM}) {
            const int64_t dk = s[0], dv = s[1];
            Tensors t = make(2, 130, 2, 4, dk, dv, GDN2_BF16, GDN2_F32, flags);
            const gdn2_problem& p = t.p;
            const int64_t tok = 2 * 130, hv = 4;
            void* dO = stub::dev_alloc(tok * hv * dv * 2);
            float* dST = static_cast<float*>(stub::dev_alloc(2 * hv * dk * dv * 4));
            void* dq = stub::dev_alloc(tok * 2 * dk * 2);
            void* dkk = stub::dev_alloc(tok * 2 * dk * 2);
            void* dvv = stub::dev_alloc(tok * hv * dv * 2);
            void* da = stub::dev_alloc(tok * hv * dk * 4);
            void* db = stub::dev_alloc(tok * hv * dk * 4);
            void* dw = stub::dev_alloc(tok * hv * dv * 4);
            float* dS0 = static_cast<float*>(stub::dev_alloc(2 * hv * dk * dv * 4));
            const size_t wsb = gdn2_chunk_bwd_workspace_size(&p);
            void* ws = stub::dev_alloc(wsb);
            auto bwd = [&](void* dqx, void* wsx, size_t n) {
                return gdn2_chunk_bwd(&p, t.q, t.k, t.v, t.alpha, t.b, t.w, t.S0, dO, dST, dqx, dkk, dvv, da, db, dw,
                                      dS0, wsx, n, nullptr);
            };
            expect("bwd valid", bwd(dq, ws, wsb), GDN2_OK, 3, 1000);
            expect("bwd dq over dk", bwd(dkk, ws, wsb), GDN2_ERR_ALIAS);
            expect("bwd dq over q", bwd(t.q, ws, wsb), GDN2_ERR_ALIAS);
            expect("bwd workspace short", bwd(dq, ws, wsb - 1), GDN2_ERR_WORKSPACE);
            // packed batch: 3 sequences of 40, 0 and 220 tokens, offsets in
            // (stand-in) device memory
            gdn2_problem pv = p;
            pv.B = 3;
            pv.T = 260;
            int32_t* cu = static_cast<int32_t*>(stub::dev_alloc(16));
            const size_t wsv = gdn2_chunk_bwd_varlen_workspace_size(&pv);
            if (wsv == 0) {
                std::fprintf(stderr, "FAIL bwd varlen workspace size 0\n");
                ++g_bad;
            }
            void* wsvp = stub::dev_alloc(wsv);
            float* S0v = static_cast<float*>(stub::dev_alloc(3 * hv * dk * dv * 4));
            float* dSTv = static_cast<float*>(stub::dev_alloc(3 * hv * dk * dv * 4));
            float* dS0v = static_cast<float*>(stub::dev_alloc(3 * hv * dk * dv * 4));
            auto bv = [&](const gdn2_problem* pp, const int32_t* c, void* dqx, size_t n) {
                return gdn2_chunk_bwd_varlen(pp, c, t.q, t.k, t.v, t.alpha, t.b, t.w, S0v, dO, dSTv, dqx, dkk, dvv,
                                             da, db, dw, dS0v, wsvp, n, nullptr);
            };
            expect("bwd varlen valid", bv(&pv, cu, dq, wsv), GDN2_OK, 4, 1000);
            expect("bwd varlen workspace short", bv(&pv, cu, dq, wsv - 1), GDN2_ERR_WORKSPACE);
            expect("bwd varlen offsets over dq", bv(&pv, reinterpret_cast<const int32_t*>(dq), dq, wsv),
                   GDN2_ERR_ALIAS);
            expect("bwd varlen offsets misaligned",
                   bv(&pv, reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(cu) + 2), dq, wsv),
                   GDN2_ERR_ALIGN);
            // no tokens: the plan and the reverse pass (dS_T through to dS0)
            gdn2_problem p0 = pv;
            p0.T = 0;
            expect("bwd varlen no tokens", bv(&p0, cu, dq, gdn2_chunk_bwd_varlen_workspace_size(&p0)), GDN2_OK, 2, 2);
            expect("bwd varlen null offsets", bv(&pv, nullptr, dq, wsv), GDN2_ERR_NULL);
        }
    }
}

void conv_cases()
{
    const int64_t B = 2, T = 70, C = 96;
    for (int io = 0; io < 2; ++io) {
        const int64_t es = io ? 2 : 4;
        void* x = stub::dev_alloc(B * T * C * es);
        void* y = stub::dev_alloc(B * T * C * es);
        float* wt = static_cast<float*>(stub::dev_alloc(C * 4 * 4));
        void* sin = stub::dev_alloc(B * 3 * C * es);
        void* sout = stub::dev_alloc(B * 3 * C * es);
        expect("conv valid", gdn2_short_conv(B, T, C, 4, GDN2_CONV_SILU, io, x, wt, sin, y, sout, nullptr), GDN2_OK, 1, 1000);
        expect("conv y over x", gdn2_short_conv(B, T, C, 4, 0, io, x, wt, sin, x, sout, nullptr), GDN2_ERR_ALIAS);
        expect("conv K 0", gdn2_short_conv(B, T, C, 0, 0, io, x, wt, sin, y, sout, nullptr), GDN2_ERR_SHAPE);
        expect("conv flag 2", gdn2_short_conv(B, T, C, 4, 2, io, x, wt, sin, y, sout, nullptr), GDN2_ERR_SHAPE);
        void* dy = stub::dev_alloc(B * T * C * es);
        void* dx = stub::dev_alloc(B * T * C * es);
        float* dwt = static_cast<float*>(stub::dev_alloc(C * 4 * 4));
        void* dsin = stub::dev_alloc(B * 3 * C * es);
        void* dsout = stub::dev_alloc(B * 3 * C * es);
        const size_t wsb = gdn2_short_conv_bwd_workspace_size(B, T, C, 4);
        void* ws = stub::dev_alloc(wsb);
        auto cb = [&](void* dxx, size_t n) {
            return gdn2_short_conv_bwd(B, T, C, 4, GDN2_CONV_SILU, io, x, wt, sin, dy, dsout, dxx, dwt, dsin, ws, n,
                                       nullptr);
        };
        expect("conv bwd valid", cb(dx, wsb), GDN2_OK, 1, 1000);
        expect("conv bwd no dstate_out",
               gdn2_short_conv_bwd(B, T, C, 4, 0, io, x, wt, sin, dy, nullptr, dx, dwt, dsin, ws, wsb, nullptr), GDN2_OK,
               1, 1000);
        expect("conv bwd dstate over dstate_out",
               gdn2_short_conv_bwd(B, T, C, 4, 0, io, x, wt, sin, dy, dsout, dx, dwt, dsout, ws, wsb, nullptr),
               GDN2_ERR_ALIAS);
        expect("conv bwd dx over dy", cb(dy, wsb), GDN2_ERR_ALIAS);
        expect("conv bwd workspace short", cb(dx, wsb - 1), GDN2_ERR_WORKSPACE);
    }
    // sizes at and past the limits
    (void)gdn2_short_conv_bwd_workspace_size(INT64_MAX, INT64_MAX, INT64_MAX, 4);
    (void)gdn2_short_conv_bwd_workspace_size(-1, 10, 10, 4);
}

void query_cases()
{
    for (int s = -3; s < 12; ++s)
        if (gdn2_status_str(s) == nullptr) {
            std::fprintf(stderr, "FAIL status_str(%d) is NULL\n", s);
            ++g_bad;
        }
    if (gdn2_abi_version() != GDN2_ABI_VERSION) ++g_bad;
    gdn2_problem p{INT64_MAX, INT64_MAX, INT64_MAX, 128, 256, 64, 1, 1, 0, INT64_MAX};
    const size_t sizes[] = {gdn2_chunk_fwd_workspace_size(&p), gdn2_chunk_prep_workspace_size(&p),
                            gdn2_chunk_fwd_varlen_workspace_size(&p), gdn2_chunk_bwd_workspace_size(&p),
                            gdn2_chunk_fwd_workspace_size(nullptr)};
    for (size_t z : sizes)
        if (z != 0) {
            std::fprintf(stderr, "FAIL workspace size of an out-of-range problem is %zu\n", z);
            ++g_bad;
        }
}

}  // namespace

int main()
{
    chunk_forward_cases();
    recurrent_cases();
    varlen_cases();
    fused_conv_cases();
    backward_cases();
    conv_cases();
    query_cases();
    const int stub_failures = stub::failures();
    std::printf("api driver: %d failed cases, %d launch-argument failures\n", g_bad, stub_failures);
    return (g_bad == 0 && stub_failures == 0) ? 0 : 1;
}
