// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

// Gates (alpha, b, w) are fp32 or bf16 as the launch's gate type says;
// flags are the GDN2_FLAG_* prologue options.  H counts value heads (one
// state each); Hk the query/key heads, H a multiple of Hk, value head h
// reading q/k head h / (H / Hk).
//
// Packed variable-length batches: B is the number of sequences, T the
// packed token count, and `plan` (null for equal-length batches) points at
// the table k_varlen_plan writes: clamped offsets cu[B+1], each sequence's
// first chunk first[B+1] (first[B] = chunk count), then per chunk its
// {first token, length}.  Chunk c of value head h owns workspace block
// h * ncmax + c; ncmax bounds the chunk count.
struct PrepArgs {
    const void* q; const void* k; const void* v;
    const void* alpha; const void* b; const void* w;
    void* ws; int64_t ws_block;
    int64_t B, T, H, Hk; int dv; int nt; int flags;
    const int* plan; int64_t ncmax;
    int64_t t_off;          // backward: byte offset of T in each block (0 = not written)
    // short convolution fused into the prologue (equal-length batches): conv_w
    // [conv_C][conv_K] fp32 over the concatenated channels q | k | v (q/k head
    // h channel c = h*DK + c and Hk*DK + h*DK + c, value head h column j =
    // 2*Hk*DK + h*dv + j); conv_in [B][conv_K-1][conv_C] holds the inputs
    // before each sequence (null = zeros); conv_w null = no convolution
    const float* conv_w; const void* conv_in; int64_t conv_C; int conv_K; int conv_silu;
};

// Checkpoints (optional): the state entering every chunk, [dk][dv] per
// workspace block in fp32 (S_chk) or in the I/O dtype (S_chkIo), and its
// transpose in the I/O dtype, S_chkT [dv][dk] per block; each may be null.
// o may be null when only states are wanted.
struct StateArgs {
    const void* ws; int64_t ws_block;
    const float* S0; void* o; float* S_out;
    int64_t B, T, H; int dv; int nt; int nslices;
    const int* plan; int64_t ncmax;
    float* S_chk; void* S_chkT; void* S_chkIo;
    // the fused short convolution's carried window: the first slice of each
    // chain writes conv_out [B][conv_K-1][conv_C] = the last conv_K-1 inputs
    // (from cq/ck/cv and conv_in, as PrepArgs) of its value head's columns,
    // and of its query/key head when it is the group's first value head
    const void* cq; const void* ck; const void* cv; const void* conv_in; void* conv_out;
    int64_t conv_C, Hk; int conv_K;
};

// cu (null for equal-length batches): the N+1 caller offsets of a packed
// batch, each clamped into [0, T] before use
// With norm_g set (whole value rows per workgroup: nslices == 1), the output
// written to o is the layer's output step applied to the token's row,
// o / sqrt(mean(o^2) + norm_eps) * norm_w * g * sigmoid(g), g [.., Hv, dv] in
// the I/O dtype, norm_w [dv] fp32.
struct RecArgs {
    const void* q; const void* k; const void* v;
    const void* alpha; const void* b; const void* w;
    const float* S_in; void* o; float* S_out;
    int64_t B, T, H, Hk; int dv; int nslices; int flags;
    const int* cu;
    const void* norm_g; const float* norm_w; float norm_eps;
    // fused short convolution (as PrepArgs); conv_out receives the window
    // after the last token and must not overlap conv_in
    const float* conv_w; const void* conv_in; void* conv_out; int64_t conv_C; int conv_K; int conv_silu;
};

// Backward (H value heads = query/key heads; equal-length batches, or a
// packed batch through `plan` and ncmax as for the forward, each chunk's
// per-chunk arrays at its workspace block number).  Reverse state pass: per
// (sequence, head, slice of vs value columns), reads the forward workspace,
// dO and dS_T (nullable), writes the gradient each chunk's exit state
// receives, [dk][dv] per block in fp32 (dSL) and/or in the I/O dtype (dSLIo),
// each nullable, and dS0 (nullable).
struct BwdStateArgs {
    const void* ws; int64_t ws_block;
    const void* dO; const float* dS_T; float* dSL; float* dS0;
    int64_t B, T, H; int dk, dv, nt, nslices, vs;
    void* dSLT;             // optional: the same transposed, [dv][dk] per block, I/O dtype
    void* dSLIo;
    int64_t t_off;          // matrix-core pass: the blocks' backward extension (BwdExt) starts here
    const int* plan; int64_t ncmax;
};

// Per-chunk gradients: inputs, dO, the chunk entry states S_chk and exit
// gradients dSL ([dk][dv] fp32 per block); writes dq, dk, dv (I/O dtype) and
// dalpha, db, dw (gate dtype).  scratch: fp32 per workgroup.  total = the
// block count (B*H*nt, or H*ncmax with a plan).
struct GradArgs {
    const void* q; const void* k; const void* v;
    const void* alpha; const void* b; const void* w; const void* dO;
    const float* S_chk; const float* dSL;
    void* dq; void* dk_out; void* dv_out; void* dalpha; void* db; void* dw;
    float* scratch;
    int64_t B, T, H; int dk, dv, nt; int64_t total;
    const int* plan; int64_t ncmax;
};

// Matrix-core per-chunk gradients, one launch of two stages (bf16 I/O; with
// the prologue flags the gates are logits and q/k unnormalised, and the
// gradients are those of the raw inputs): the value side reads the forward
// workspace (blocks of ws_block bytes, the backward's extension at t_off),
// the checkpoints S_chk/S_chkT and dSL/dSLT (bf16, [dk][dv] and [dv][dk] per
// chunk), dO, v, w and writes dw, dv; the key side takes its results from
// LDS and reads q, k, b, alpha to write dq, dk, db, dalpha.
struct GradVArgs {
    const void* ws; int64_t ws_block, t_off;
    const void* v; const void* w; const void* dO;
    const void* S_chk; const void* S_chkT; const void* dSL; const void* dSLT;
    void* dw; void* dv_out;
    int64_t B, T, H; int dk, dv, nt; int64_t total;
    int flags;              // prologue options applied in-kernel (gradients of the logits, raw q/k)
    const int* plan; int64_t ncmax;
};

struct GradKArgs {
    const void* q; const void* k; const void* alpha; const void* b;
    void* dq; void* dk_out; void* dalpha; void* db;
    int64_t B, T, H; int dk, nt; int64_t total;
    int flags;
    const int* plan; int64_t ncmax;
};

// Prologue options in the backward.  Query/key rows (rows = B*T*Hk of dk
// channels): the pre launch writes qh, kh = the rows, L2-normalised when l2,
// each copied to the G value heads of its group ([B,T,Hk*G,dk]); the post
// launch sums dqh, dkh over the G heads and takes the sum through the norm
// (reading q, k) into dq, dk_out.  All in the I/O dtype.
struct QkMapArgs {
    const void* q; const void* k; void* qh; void* kh;
    const void* dqh; const void* dkh; void* dq; void* dk_out;
    int64_t rows; int G, dk; bool l2;
};

// Gate logits z[j] (gate dtype, n[j] elements each, a multiple of 4): the
// pre launch writes dst[j] = scale[j] * sigmoid(z) as fp32, the post launch
// dst[j] (gate dtype) = grad[j] * scale[j] * s (1 - s).
struct GateMapArgs {
    const void* z[3]; const float* grad[3]; void* dst[3];
    int64_t n[3]; float scale[3];
};

struct PlanArgs {
    const int* cu; int* plan;
    int64_t N, T, ncmax;
};

struct NormArgs {
    const void* o; const void* g; const float* weight; void* y;
    int64_t rows; int dv; float inv_dv; float eps;
};

// short convolution: a workgroup takes 256 channels of a span of tokens
// staged through LDS; forward spans of kConvSpanF(bf16) tokens, backward
// workgroups of kConvSpan tokens that each write one fp32 [C][K] row of
// weight partials
constexpr int kConvSpan = 128;
constexpr int kConvSpanF(bool bf16) { return bf16 ? 64 : 32; }

struct ConvArgs {
    const void* x; const float* weight; const void* state_in; void* y; void* state_out;
    int64_t B, T, C;
    int64_t ntile;        // forward spans a sequence (at least 1 when the state is written)
};

struct ConvBwdArgs {
    const void* x; const float* weight; const void* state_in; const void* dy;
    void* dx; float* dweight; void* dstate; float* part;
    const void* dstate_out;   // gradient of the window after the last token (null = zeros)
    int64_t B, T, C;
    int64_t nspan;        // spans a sequence (at least 1)
};

// Each returns hipSuccess or the launch error.  bf16 selects the I/O dtype,
// gbf16 the gate dtype (bf16 gates only with bf16 I/O).
hipError_t launch_chunk_prep(const PrepArgs& a, int dk, bool bf16, bool gbf16, hipStream_t s);
hipError_t launch_chunk_state(const StateArgs& a, int dk, int vs, bool bf16, hipStream_t s);
hipError_t launch_recurrent(const RecArgs& a, int dk, int vs, bool bf16, bool gbf16, hipStream_t s);

hipError_t launch_gated_rmsnorm(const NormArgs& a, bool bf16, hipStream_t s);
hipError_t launch_short_conv(const ConvArgs& a, int K, bool silu, bool bf16, hipStream_t s);
// the gradient launch, then the fixed-order sum of the weight partials
hipError_t launch_short_conv_bwd(const ConvBwdArgs& a, int K, bool silu, bool bf16, hipStream_t s);
hipError_t launch_varlen_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_chunk_state_bwd(const BwdStateArgs& a, bool bf16, hipStream_t s);
// the same on the matrix-core path (bf16, dk in {32, 64, 128}, dv in {32, 64,
// 128}, slices of 32): blocks in the backward's layout, dSLIo and dSLT only
hipError_t launch_chunk_state_bwd_mf(const BwdStateArgs& a, hipStream_t s);
int state_bwd_slice(int dv);
hipError_t launch_bwd_qk_map(const QkMapArgs& a, bool post, bool bf16, hipStream_t s);
hipError_t launch_bwd_gate_map(const GateMapArgs& a, bool post, bool gbf16, hipStream_t s);
hipError_t launch_chunk_grad(const GradArgs& a, bool bf16, bool gbf16, hipStream_t s);
hipError_t launch_chunk_grad_mf(const GradVArgs& v, const GradKArgs& k, bool gbf16, hipStream_t s);
bool gradmf_supported(int dk, int dv, bool bf16);
// workgroups of the gradient launch and the bytes of its scratch
int64_t grad_blocks(int64_t total);
int64_t chunk_grad_scratch_bytes(int dk, int dv, int64_t total);

// gdn2_chunk_fwd_noalloc's workspace: the device address of the current
// device's copy of the library's fixed scratch array (GDN2_NOALLOC_SCRATCH_BYTES),
// looked up once per device; nullptr when there is no usable device.
void* noalloc_scratch();

// int32 words of the varlen plan ahead of its chunk table (kept even so the
// 8-byte table entries stay aligned)
__host__ __device__ inline int64_t plan_head_words(int64_t N) { return 2 * (N + 1); }

// Value-slice width the state pass uses for a problem (16, 32 or 64).
int chunk_state_slice(int64_t nchains, int dv, int dk, int esize);
// Value-slice width the recurrent kernel uses (16, 32, 64 or 128).
int recurrent_slice(int64_t nchains, int64_t T, int dv);

}  // namespace gdn2
