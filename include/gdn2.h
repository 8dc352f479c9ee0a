/*
 * gdn2.h -- C ABI of the Gated DeltaNet-2 token-mixer core for AMD MI355X (gfx950).
 *
 * The core computes, per (batch, head), the recurrence on a fp32 matrix state
 * S of shape (dk, dv) given in the burn-gdn2 0.1.9 README (docs.rs), section
 * "Architecture":
 *
 *     S_t = (I - k_t (b_t * k_t)^T) diag(alpha_t) S_{t-1} + k_t (w_t * v_t)^T
 *     o_t = q_t^T S_t
 *
 * alpha (decay) and b (erase gate) are per key channel, w (write gate) per
 * value channel.  The output reads the state after the token's update; there
 * is no query scale.  By default q, k and the gates enter the core as given
 * (the layer L2-normalises q and k and activates the gates before it, README
 * "Architecture" diagram); the flags below move those prologue steps into
 * the kernels.
 *
 * Two forward modes (README intro and "Architecture"): a chunked WY form used
 * for training-length sequences (chunk size 64, README "Configuration") and a
 * fused token-by-token recurrent form used for inference with a persistent
 * state (README "Quick start").  Both compute the same function; only the
 * rounding differs.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every pointer is device memory owned by the caller.  The library
 *   never allocates, frees or synchronises, keeps no mutable global state, and
 *   launches all work on `stream` (a hipStream_t; NULL = the default stream).
 *   Calls on different streams are independent if their outputs and
 *   workspaces are disjoint.
 * Layouts (all C-contiguous, element strides implied by the sizes):
 *   q, k           : [B, T, H,  dk]
 *   alpha, b       : [B, T, Hv, dk]
 *   v, w, o        : [B, T, Hv, dv]
 *   S0/S_in, S_out : [B, Hv, dk, dv]   fp32, dv fastest
 *   with Hv = p->Hv value heads (0 = H).  Grouped value heads (README
 *   "Configuration": num_v_heads, "None = same as num_heads"): Hv a multiple
 *   of H, and value head hv reads query/key head hv / (Hv / H).  Each value
 *   head has its own state, gates and values; only q and k are shared.
 * Dtypes.  io_dtype covers q, k, v and o; gate_dtype covers alpha, b, w.
 *   Supported pairs: (GDN2_F32, GDN2_F32), (GDN2_BF16, GDN2_F32) and
 *   (GDN2_BF16, GDN2_BF16).  The state is always fp32; all arithmetic is
 *   fp32 (bf16 only as matrix-core operands).  bf16 outputs are rounded to
 *   nearest even.
 * Prologue flags (gdn2_problem.flags, any combination of):
 *   GDN2_FLAG_GATE_LOGITS  alpha, b, w hold pre-activation values; the
 *       kernels use sigmoid(alpha), sigmoid(b), sigmoid(w), sigmoid(x) =
 *       1 / (1 + exp(-x)).  (The README names the gate projections but not
 *       their activation; the sigmoid is this library's reading.)
 *   GDN2_FLAG_NEG_EIGVAL   with GATE_LOGITS only: b = 2 * sigmoid(b), the
 *       README's allow_neg_eigval option ("b x 2", "Configuration").
 *   GDN2_FLAG_QK_L2NORM    q and k are L2-normalised per (token, head) over
 *       dk inside the kernels, x / sqrt(sum(x^2) + 1e-6) (README
 *       "Architecture": L2-Norm before the recurrence).
 *   Any other bit, or NEG_EIGVAL without GATE_LOGITS, is GDN2_ERR_SHAPE.
 * Sizes.  B, T, H >= 0 (any zero makes the call a no-op apart from the
 *   state copy described below); Hv = 0 or a positive multiple of H; dk in
 *   {16, 32, 64, 128}; dv a multiple of 16 in [16, 256]; chunk == 64 for the
 *   chunked mode.
 * Domain.  alpha in [0, 1] (after the sigmoid with GATE_LOGITS).  The
 *   chunked forward rescales keys and queries by decay products of at most
 *   4 consecutive tokens (and their inverses), so it raises every alpha
 *   below 2^-20 (zero included) to 2^-20: those products then stay >= 2^-80
 *   and their inverses finite, and a raised decay keeps at most a 2^-20
 *   share of the state it should have erased (a relative change far below
 *   either parity bar); every other decay factor it forms is a product of
 *   alphas (<= 1), so fast decay only underflows negligible terms.  The
 *   chunked backward raises alpha the same way and returns the gradient of
 *   that forward: where alpha < 2^-20 the forward does not depend on alpha,
 *   and dalpha (d logit with GATE_LOGITS) is 0 there.
 *   The recurrent mode uses alpha as given.  b, w, q, k, v are any finite
 *   values (b in (0, 2) is the README's negative-eigenvalue option, "b x 2").
 * Alignment.  Every tensor pointer is 16-byte aligned (the kernels use
 *   16-byte vector accesses); the workspace is 256-byte aligned (a workspace
 *   that is not is GDN2_ERR_WORKSPACE).
 * Aliasing.  Inputs are never written.  Outputs (o, S_out, workspace) must
 *   not overlap any input or each other, except that S_out may equal S0 /
 *   S_in exactly (in-place state update).  Any other overlap is an error.
 * Errors.  Every argument is checked on the host before anything is
 *   launched; the first failing check returns its code and nothing runs.
 *   A failed launch returns GDN2_ERR_DEVICE (also when no GPU is present).
 *   Faults inside a kernel surface on the stream, as for any HIP launch.
 *   Nothing is printed and no C++ exception crosses this interface.
 */
#ifndef GDN2_H_
#define GDN2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN2_ABI_VERSION 8

typedef enum {
    GDN2_OK = 0,
    GDN2_ERR_NULL = 1,       /* a required pointer is NULL                      */
    GDN2_ERR_SHAPE = 2,      /* unsupported or inconsistent sizes               */
    GDN2_ERR_DTYPE = 3,      /* unsupported dtype pair                          */
    GDN2_ERR_ALIAS = 4,      /* an output overlaps an input or another output   */
    GDN2_ERR_WORKSPACE = 5,  /* workspace missing, too small or not 256-B aligned */
    GDN2_ERR_DEVICE = 6,     /* no usable GPU, or a launch failed               */
    GDN2_ERR_ALIGN = 7       /* a pointer is misaligned (16 B; cu_seqlens 4 B)  */
} gdn2_status;

typedef enum { GDN2_F32 = 0, GDN2_BF16 = 1 } gdn2_dtype;

enum {
    GDN2_FLAG_GATE_LOGITS = 1,   /* gates are pre-activations: sigmoid in-kernel */
    GDN2_FLAG_NEG_EIGVAL = 2,    /* b = 2 * sigmoid(b) (requires GATE_LOGITS)     */
    GDN2_FLAG_QK_L2NORM = 4      /* L2-normalise q and k over dk in-kernel        */
};

enum { GDN2_CONV_SILU = 1 };     /* gdn2_short_conv: y = z * sigmoid(z)          */

/* Problem description (plain old data; 64 bytes). */
typedef struct {
    int64_t B, T, H;         /* batch, tokens per sequence, query/key heads   */
    int64_t dk, dv;          /* key/query width and value width of a head     */
    int32_t chunk;           /* chunk length of the chunked mode; must be 64  */
    int32_t io_dtype;        /* gdn2_dtype of q, k, v, o                      */
    int32_t gate_dtype;      /* gdn2_dtype of alpha, b, w                     */
    int32_t flags;           /* GDN2_FLAG_* prologue options (0 = none)       */
    int64_t Hv;              /* value heads: 0 (= H) or a multiple of H       */
} gdn2_problem;

/* ABI version of the loaded library (GDN2_ABI_VERSION). */
int gdn2_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* gdn2_status_str(int status);

/*
 * Bytes of device workspace gdn2_chunk_fwd needs for problem *p (0 if *p is
 * invalid).  The workspace holds, per (batch, head, chunk), the chunk's WY
 * factors and decay-scaled operands; it is scratch, its contents are
 * undefined between calls, and it must be 256-byte aligned.
 */
size_t gdn2_chunk_fwd_workspace_size(const gdn2_problem* p);

/*
 * Bytes of workspace the two stages gdn2_chunk_prep and gdn2_chunk_state
 * (declared below) need for problem *p when called on their own (0 if *p is
 * invalid); in this version the same as gdn2_chunk_fwd_workspace_size.
 */
size_t gdn2_chunk_prep_workspace_size(const gdn2_problem* p);

/*
 * Chunked forward (README: "chunked WY decomposition", chunk_size 64).
 * Computes o for all T tokens and, if S_out != NULL, the state after token
 * T-1.  S0 == NULL means the zero initial state (README "Quick start": the
 * state starts empty).  T need not be a multiple of 64.
 *
 * Runs as two launches on `stream`: gdn2_chunk_prep followed by
 * gdn2_chunk_state (declared below), which callers may also issue
 * themselves, e.g. to time them apart.  One case differs: a single long
 * sequence whose state pass would leave most of the GPU idle (B == 1, at
 * least 256 chunks, few value heads) with S_out != NULL, on a stream that is
 * not being captured, runs in pieces of 32 chunks (at most 256), the prep of
 * each later piece on a second stream the library keeps per device (default
 * priority), ordered by events.  The call's work is still ordered on
 * `stream` as a whole (it starts after what `stream` already holds and
 * whatever is enqueued on `stream` afterwards sees o and S_out), results
 * are bit-identical to the two launches, and concurrent calls on one device
 * serialise their enqueueing.  Under stream capture the two launches are
 * always used.
 */
int gdn2_chunk_fwd(const gdn2_problem* p,
                   const void* q, const void* k, const void* v,
                   const void* alpha, const void* b, const void* w,
                   const float* S0, void* o, float* S_out,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * First stage of gdn2_chunk_fwd, fully parallel over (batch, head, chunk):
 * forms each chunk's cumulative key-axis decay, its erase-interaction matrix
 * and the WY factors (unit-lower-triangular solve), and writes them with the
 * decay-scaled q/k operands into `workspace`.  Reads q, k, v, alpha, b, w.
 */
int gdn2_chunk_prep(const gdn2_problem* p,
                    const void* q, const void* k, const void* v,
                    const void* alpha, const void* b, const void* w,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Second stage of gdn2_chunk_fwd: the sequential pass over chunks that
 * carries the fp32 state of every (batch, head) and writes o and S_out.
 * Reads only the workspace written by gdn2_chunk_prep for the same problem,
 * and S0.
 */
int gdn2_chunk_state(const gdn2_problem* p, const float* S0, void* o, float* S_out,
                     const void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn2_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same computation, arguments (minus the workspace), checks and launches as
 * gdn2_chunk_fwd; the workspace is a fixed device array inside the library
 * (GDN2_NOALLOC_SCRATCH_BYTES, 64 MiB on every GPU the library runs on, held
 * until the process ends), so the call allocates nothing.  A problem whose
 * workspace (gdn2_chunk_fwd_workspace_size) is larger returns
 * GDN2_ERR_WORKSPACE before anything runs; d128 bf16 needs 1,160 bytes per
 * (token, value head), e.g. B1 T2048 H16 = 38 MB.  All calls on one GPU share
 * that GPU's array: calls whose work overlaps in time on one GPU (other
 * streams, other threads) race and give undefined results; calls in one
 * stream's order are safe.  Nothing in the array needs to start at zero.
 */
#define GDN2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int gdn2_chunk_fwd_noalloc(const gdn2_problem* p,
                           const void* q, const void* k, const void* v,
                           const void* alpha, const void* b, const void* w,
                           const float* S0, void* o, float* S_out, void* stream);

/*
 * Fused recurrent forward (README: "Fused Recurrent", token-by-token
 * inference with a persistent state).  Processes the T tokens one after the
 * other from S_in (NULL = zero state), writes o for each token and, if
 * S_out != NULL, the final state.  T == 1 is the decode step; passing
 * S_out == S_in updates the state in place.  p->chunk is ignored.
 */
int gdn2_recurrent_step(const gdn2_problem* p,
                        const void* q, const void* k, const void* v,
                        const void* alpha, const void* b, const void* w,
                        const float* S_in, void* o, float* S_out, void* stream);

/*
 * The recurrent forward with the layer's output step fused into its output
 * write (README "Architecture": the core's output passes through "Gated RMS
 * Norm <- SiLU Gate"; "Configuration": norm_eps = 1e-5): for every token and
 * value head, with o the row gdn2_recurrent_step would write,
 *
 *     y = o / sqrt(mean(o^2) + 1e-5) * norm_weight * g * sigmoid(g)
 *
 * (the reading of gdn2_gated_rmsnorm below), computed from o in fp32 before
 * it is rounded.  One workgroup holds whole value rows, so dv must be one of
 * 16, 32, 64, 128, 256 (else GDN2_ERR_SHAPE).  g: [B, T, Hv, dv] io_dtype,
 * norm_weight: [dv] fp32, y: [B, T, Hv, dv] io_dtype.  Everything else
 * (sizes, dtypes, flags, grouped heads, S_in/S_out, in-place state, checks)
 * is as for gdn2_recurrent_step; y must not overlap any input.  T == 1 is
 * the decode step with its output step, one launch, the layer's o never
 * written to memory.
 */
int gdn2_recurrent_step_gated(const gdn2_problem* p,
                              const void* q, const void* k, const void* v,
                              const void* alpha, const void* b, const void* w,
                              const float* S_in, const void* g, const float* norm_weight,
                              void* y, float* S_out, void* stream);

/*
 * Packed variable-length batches.  The recurrence runs per sequence and each
 * sequence starts from its own state (README "Architecture" and "Quick
 * start"); a packed batch lays N sequences back to back on the token axis
 * so that sequences of different lengths share one call without padding.
 *   p->B      = N, the number of sequences;
 *   p->T      = the total number of packed tokens (< 2^31);
 *   cu_seqlens: N+1 int32 token offsets in device memory (4-byte aligned,
 *               read by the kernels, never written): sequence i holds tokens
 *               cu_seqlens[i] .. cu_seqlens[i+1]-1; the offsets must rise
 *               from cu_seqlens[0] = 0 to cu_seqlens[N] = T (equal
 *               neighbours are empty sequences, whose state passes through).
 * Layouts: q, k [T, H, dk]; alpha, b [T, Hv, dk]; v, w, o [T, Hv, dv];
 * S0/S_in, S_out [N, Hv, dk, dv].  Everything else (dtypes, flags, grouped
 * value heads, alignment, aliasing, in-place state) is as for the calls
 * above; cu_seqlens counts as an input for the aliasing rule.
 * The offsets live on the device, so the host cannot check them: offsets
 * that break the rule give undefined o and S_out, but every offset is
 * clamped into [0, T] (and, in the chunked mode, to at least its
 * predecessor) before use, so no access leaves the tensors.
 *
 * Chunked mode: each sequence's chunks start at its first token (no chunk
 * spans two sequences).  Three launches on `stream`: a one-workgroup plan
 * (per-chunk token ranges, written into the workspace), the prep stage and
 * the state pass.
 */
size_t gdn2_chunk_fwd_varlen_workspace_size(const gdn2_problem* p);

int gdn2_chunk_fwd_varlen(const gdn2_problem* p, const int32_t* cu_seqlens,
                          const void* q, const void* k, const void* v,
                          const void* alpha, const void* b, const void* w,
                          const float* S0, void* o, float* S_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Fused recurrent mode over a packed batch: one pass per sequence. */
int gdn2_recurrent_varlen(const gdn2_problem* p, const int32_t* cu_seqlens,
                          const void* q, const void* k, const void* v,
                          const void* alpha, const void* b, const void* w,
                          const float* S_in, void* o, float* S_out, void* stream);

/*
 * Backward pass of the chunked forward (README: chunk mode is the training
 * mode).  For the loss  sum(dO * o) + sum(dS_T * S_T)  of the forward
 * gdn2_chunk_fwd(p, q, k, v, alpha, b, w, S0) computes its gradients with
 * respect to every input, in the forward's layout:
 *   dq, dk            [B, T, H, dk]      io_dtype
 *   dv                [B, T, Hv, dv]     io_dtype
 *   dalpha, db, dw    [B, T, Hv, dk|dv]  gate_dtype
 *   dS0               [B, Hv, dk, dv]    fp32 (NULL: not wanted)
 * dO [B, T, Hv, dv] (io_dtype) is the gradient of o; dS_T (fp32, NULL = 0)
 * that of the final state; S0 NULL = the zero initial state, as in the
 * forward.  Every prologue flag and grouped value heads (README,
 * "Architecture" and "Configuration") are supported: with gate logits the
 * gradients are those of the logits, with the L2 norm those of the raw q
 * and k, and a query/key head shared by G value heads gets the sum of their
 * gradients.
 * The forward is recomputed inside (no forward workspace is kept between
 * the calls); the backward is exact up to rounding, with fp32 accumulation
 * throughout and the matrix-product operands in io_dtype (with bf16 I/O the
 * chunk checkpoints and the per-chunk values handed between the gradient
 * stages are kept in bf16 too).
 * Every gradient output must be distinct from every input and from each
 * other (GDN2_ERR_ALIAS); all tensors 16-byte aligned; the workspace
 * 256-byte aligned and at least gdn2_chunk_bwd_workspace_size(p) bytes (it
 * holds the forward factors, the state entering every chunk, the state
 * gradient leaving every chunk, per-chunk scratch and, where the options
 * are mapped outside the kernels, the mapped inputs and their gradients).
 * Launches four kernels on `stream` with bf16 I/O and dk, dv in
 * {32, 64, 128} (forward recompute, checkpointing state pass, reverse pass,
 * per-chunk gradients), five otherwise.  On that path the kernels apply
 * the prologue options themselves; grouped
 * heads then add one kernel before and one after (q/k widened to the value
 * heads, their gradients summed per group).  Other shapes map every option
 * that way: one kernel before and one after for the q/k rows (L2 norm or
 * grouped heads) and for the gates (logits).
 */
size_t gdn2_chunk_bwd_workspace_size(const gdn2_problem* p);

int gdn2_chunk_bwd(const gdn2_problem* p,
                   const void* q, const void* k, const void* v,
                   const void* alpha, const void* b, const void* w,
                   const float* S0, const void* dO, const float* dS_T,
                   void* dq, void* dk, void* dv, void* dalpha, void* db, void* dw, float* dS0,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of gdn2_chunk_fwd_varlen (packed batches, layouts, p->B = N,
 * p->T = total tokens and cu_seqlens in DEVICE memory exactly as for that
 * call, the same offsets clamped the same way).  The gradients and their
 * meaning are those of gdn2_chunk_bwd, per sequence: dq, dk, dalpha, db,
 * dw, dv in the packed layouts of the inputs, dS0 [N, Hv, dk, dv] (NULL =
 * not wanted); S0 and dS_T [N, Hv, dk, dv] or NULL (zero).  An empty
 * sequence passes its dS_T through to dS0.
 * The whole batch runs in the launches of gdn2_chunk_bwd plus the
 * one-workgroup plan of gdn2_chunk_fwd_varlen, written into the head of the
 * workspace: every per-chunk kernel takes one workgroup per (value head,
 * chunk slot) and finds its sequence and tokens in the plan, and every
 * state pass one workgroup per (sequence, value head, column slice), so
 * the launch count does not grow with N.  The workspace (256-byte aligned,
 * at least gdn2_chunk_bwd_varlen_workspace_size(p) bytes, which depends on
 * N and T only) holds the plan and gdn2_chunk_bwd's arrays for
 * ceil(T/64) + N chunk slots per value head.  Aliasing and alignment are
 * checked over the packed tensors as a whole; the offsets count as an
 * input.
 */
size_t gdn2_chunk_bwd_varlen_workspace_size(const gdn2_problem* p);

int gdn2_chunk_bwd_varlen(const gdn2_problem* p, const int32_t* cu_seqlens,
                          const void* q, const void* k, const void* v,
                          const void* alpha, const void* b, const void* w,
                          const float* S0, const void* dO, const float* dS_T,
                          void* dq, void* dk, void* dv, void* dalpha, void* db, void* dw, float* dS0,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Output step of the layer (README "Architecture": "Gated RMS Norm <- SiLU
 * Gate"; "Configuration": norm_eps = 1e-5).  For every (token, head) row of
 * dv channels
 *
 *     y = o / sqrt(mean(o^2) + 1e-5) * weight * g * sigmoid(g)
 *
 * with one fp32 weight vector [dv] shared by all heads (the SiLU-gate form
 * and the shared weight are this library's reading of the diagram).
 * o, g, y: [B, T, Hv, dv] in io_dtype; weight: [dv] fp32.  dk, chunk,
 * gate_dtype and flags are checked as for the other calls but unused.
 * y may equal o exactly (normalise in place); any other overlap is
 * GDN2_ERR_ALIAS.  Usable after either forward mode.  (The chunked state pass
 * splits a head's value columns over several workgroups, so the row
 * statistic cannot be taken inside its output write; this call streams o, g
 * and y once.)
 */
int gdn2_gated_rmsnorm(const gdn2_problem* p, const void* o, const void* g, const float* weight,
                       void* y, void* stream);

/*
 * Short convolution of the layer's prologue (README "Architecture": the q, k
 * and v projections pass through a "ShortConv" before the L2 norm;
 * "Configuration": use_short_conv, a depthwise convolution before the
 * recurrence).  The README gives neither the width nor the activation; this
 * library reads it as a causal depthwise convolution over tokens with K taps
 * per channel and an optional SiLU:
 *
 *     z[b,t,c] = sum_{i<K} weight[c,i] * xe[b, t-(K-1)+i, c]
 *     y = z, or z * sigmoid(z) with GDN2_CONV_SILU
 *
 * where xe reads x at positions >= 0 and, at the K-1 positions before the
 * first token, the carried state: xe[b, -(K-1)+j, c] = state_in[b, j, c]
 * (zeros when state_in is NULL).  state_out, when not NULL, receives the
 * last K-1 positions of xe (the window a following call continues from), so
 * that calls on consecutive pieces of a sequence equal one call on the whole.
 *
 * Shapes and dtypes: x, y: [B, T, C]; state_in, state_out: [B, K-1, C],
 * all in io_dtype (gdn2_dtype; the state holds inputs and is copied
 * exactly); weight: [C, K] fp32.  All arithmetic is fp32.  B, T >= 0,
 * C > 0 a multiple of 8, 1 <= K <= 8 (with K == 1 the state pointers are
 * ignored); flags is 0 or GDN2_CONV_SILU.  A concatenated [B, T, C] tensor
 * of the q, k and v projections is convolved in one call.
 * Aliasing: y must not overlap any input (tiles read their neighbours'
 * inputs); state_out may equal state_in exactly (in-place update), any
 * other overlap is GDN2_ERR_ALIAS.  16-byte alignment, errors, streams and
 * ownership as for every other call.  One launch on `stream`.
 */
int gdn2_short_conv(int64_t B, int64_t T, int64_t C, int32_t K, int32_t flags, int32_t io_dtype,
                    const void* x, const float* weight, const void* state_in,
                    void* y, void* state_out, void* stream);

/*
 * Bytes of workspace gdn2_short_conv_bwd needs (0 for invalid sizes): one
 * fp32 [C, K] row of partial weight gradients per (sequence, 128-token span).
 */
size_t gdn2_short_conv_bwd_workspace_size(int64_t B, int64_t T, int64_t C, int32_t K);

/*
 * Gradient of gdn2_short_conv given dy = dL/dy (same shapes, dtypes and
 * flags; state_in as in the forward, NULL = zeros):
 *
 *     dz = dy, or dy * s * (1 + z * (1 - s)), s = sigmoid(z)   (SiLU)
 *     dxe[b,p,c] = sum_i weight[c,i] * dz[b, p+(K-1)-i, c]  over 0 <= p+(K-1)-i < T
 *     dweight[c,i] = sum_{b,t} dz[b,t,c] * xe[b, t-(K-1)+i, c]
 *
 * dstate_out [B, K-1, C] (io_dtype; NULL = zeros) is the gradient with
 * respect to the forward's state_out, the last K-1 positions of xe: it is
 * added to dxe there, so that a sequence processed in pieces is
 * differentiated piece by piece, last first, each piece's dstate_in handed
 * to the piece before it as dstate_out (the pieces' dweight summed).
 * dx = dxe at positions >= 0; dstate_in (NULL = not wanted) = dxe at the K-1
 * positions before the first token, the gradient with respect to state_in
 * (also when state_in is NULL, i.e. zero).  dx, dstate_in: io_dtype; dweight: fp32 [C, K], summed in a
 * fixed order (the result does not depend on scheduling).  Outputs and the
 * workspace (16-byte aligned, at least gdn2_short_conv_bwd_workspace_size
 * bytes) must not overlap any input or each other.  Two launches on `stream`
 * (gradients with per-span weight partials, then the fixed-order sum).
 */
int gdn2_short_conv_bwd(int64_t B, int64_t T, int64_t C, int32_t K, int32_t flags, int32_t io_dtype,
                        const void* x, const float* weight, const void* state_in, const void* dy,
                        const void* dstate_out, void* dx, float* dweight, void* dstate_in,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The short convolution fused into the core's prologue (README "Architecture":
 * the projections pass through the ShortConv, then the L2 norm, into the
 * recurrence; "Configuration": use_short_conv).  The two calls below compute
 * exactly what gdn2_short_conv on the concatenated projection followed by
 * gdn2_chunk_fwd / gdn2_recurrent_step on its three parts computes, in one
 * pass that writes no convolved tensor:
 *
 *   x = [q | k | v] per token, C = 2 H dk + Hv dv channels: query/key head h
 *       channel c of q is h dk + c, of k is H dk + h dk + c; value head h
 *       column j of v is 2 H dk + h dv + j;
 *   (q', k', v') = gdn2_short_conv(x, weight, state_in, flags), each rounded
 *       to io_dtype as that call stores it;
 *   o, S_out as the core computes them from q', k', v' and the gates.
 *
 * weight [C, K] fp32 and the windows [B, K-1, C] (io_dtype) have the layout
 * gdn2_short_conv takes for the concatenated projection, so a caller can move
 * between the two forms.  1 <= K <= 4; flags 0 or GDN2_CONV_SILU; with K == 1
 * the window pointers are ignored.  state_in NULL = zeros; state_out NULL =
 * not written.  Equal-length batches only (no packed-batch form).  Everything
 * else (sizes, dtypes, flags of the problem, alignment, errors, streams) is as
 * for the unfused calls; weight and the windows count as inputs and outputs
 * for the aliasing rule.
 */
typedef struct {
    const float* weight;     /* [C, K] fp32                                    */
    const void* state_in;    /* [B, K-1, C] io_dtype, or NULL (zeros)           */
    void* state_out;         /* [B, K-1, C] io_dtype, or NULL (not written)     */
    int32_t K;               /* taps, 1..4                                       */
    int32_t flags;           /* 0 or GDN2_CONV_SILU                              */
} gdn2_conv;

/*
 * gdn2_chunk_fwd with the fused convolution.  Same workspace
 * (gdn2_chunk_fwd_workspace_size) and two launches; state_out may equal
 * state_in exactly (the window is written by the second launch, after the
 * first has read every input it needs).
 */
int gdn2_chunk_fwd_conv(const gdn2_problem* p, const gdn2_conv* conv,
                        const void* q, const void* k, const void* v,
                        const void* alpha, const void* b, const void* w,
                        const float* S0, void* o, float* S_out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn2_recurrent_step with the fused convolution (T == 1: the decode step
 * with its convolution window).  One launch.  state_out must not overlap
 * state_in (GDN2_ERR_ALIAS): the workgroups of one sequence read the window
 * while the first of them writes the next one, so a serving loop alternates
 * two window buffers.
 */
int gdn2_recurrent_step_conv(const gdn2_problem* p, const gdn2_conv* conv,
                             const void* q, const void* k, const void* v,
                             const void* alpha, const void* b, const void* w,
                             const float* S_in, void* o, float* S_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H_ */
