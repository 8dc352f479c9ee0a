"""fp64 CPU oracle for the Gated DeltaNet-2 token mixer (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it.

What is computed
----------------
The per-head recurrence on a matrix state S of shape (d_k, d_v), as written in
the burn-gdn2 0.1.9 README (docs.rs), section "Architecture" (the per-token
recurrence block):

    S_t = (I - k_t (b_t * k_t)^T) diag(alpha_t) S_{t-1} + k_t (w_t * v_t)^T
    o_t = q_t^T S_t

alpha (decay) and b (erase gate) act per key channel, w (write gate) per value
channel; the Gated DeltaNet-2 explainer (asapai.co.kr), section on splitting
the single gate into two knobs, describes the same three per-channel gates.

Readings taken where the page leaves a step open (each also listed in the
design notes of the repository):
  * the output reads the state *after* this token's update (S_t);
  * the decay is applied first, the erase reads the decayed state;
  * the erase subtracts along k and reads with b*k (literal order of the
    product k (b*k)^T);
  * no 1/sqrt(d_k) query scale, no normalisation inside the core;
  * a missing initial state means S_0 = 0 (the README's quick start starts
    inference from an empty state).

Layouts (all row-major / C-contiguous):
  q, k, alpha, b : [B, T, H, d_k]
  v, w           : [B, T, H, d_v]
  S0, S          : [B, H, d_k, d_v]
  o              : [B, T, H, d_v]
(with grouped value heads, H here is the value-head count: ``share_qk_heads``
widens q and k to it first).

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
hand-worked examples (``tests/golden``), the special cases the pages name
(KDA, Gated DeltaNet, plain linear attention), exact-recall and
Householder invariants, and against each other.
"""
from __future__ import annotations

import numpy as np

__all__ = ["recurrent", "chunked_wy", "rel_l2", "rel_l2_chains", "prologue", "sigmoid", "gated_rmsnorm", "NORM_EPS", "share_qk_heads", "varlen",
           "FLAG_GATE_LOGITS", "FLAG_NEG_EIGVAL", "FLAG_QK_L2NORM", "short_conv", "short_conv_bwd", "CONV_SILU"]

# prologue options (the library's GDN2_FLAG_* values)
FLAG_GATE_LOGITS, FLAG_NEG_EIGVAL, FLAG_QK_L2NORM = 1, 2, 4
L2NORM_EPS = 1e-6


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def sigmoid(x):
    """Logistic function 1 / (1 + exp(-x)), fp64."""
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def prologue(q, k, alpha, b, w, flags=0):
    """The steps the layer runs right before the core, as optional flags.

    burn-gdn2 README, "Architecture" diagram: the Q/K/V/B/W/G projections are
    followed by L2-Norm before the recurrence, and "Configuration" lists
    allow_neg_eigval ("b x 2").  The README does not name the gate activation;
    the logistic sigmoid is the reading taken here (the synthetic workloads
    draw their gates as sigmoids of normal logits).

      FLAG_GATE_LOGITS: alpha, b, w are pre-activations -> sigmoid(.)
      FLAG_NEG_EIGVAL (with GATE_LOGITS): b -> 2 * sigmoid(b)
      FLAG_QK_L2NORM: q, k -> x / sqrt(sum over d_k of x^2 + 1e-6), per row

    Returns fp64 (q, k, alpha, b, w), ready for ``recurrent``/``chunked_wy``.
    """
    q, k, alpha, b, w = map(_f64, (q, k, alpha, b, w))
    if flags & FLAG_NEG_EIGVAL and not flags & FLAG_GATE_LOGITS:
        raise ValueError("NEG_EIGVAL needs GATE_LOGITS")
    if flags & FLAG_GATE_LOGITS:
        alpha = sigmoid(alpha)
        b = sigmoid(b) * (2.0 if flags & FLAG_NEG_EIGVAL else 1.0)
        w = sigmoid(w)
    if flags & FLAG_QK_L2NORM:
        q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + L2NORM_EPS)
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + L2NORM_EPS)
    return q, k, alpha, b, w


def share_qk_heads(q, k, Hv):
    """Grouped value heads (burn-gdn2 README, "Configuration": num_v_heads, whose
    default is the number of query/key heads).

    With Hv value heads over H query/key heads (Hv a multiple of H, G = Hv / H),
    each value head keeps its own state, gates and values and reads the q and
    k of one query/key head.  The README does not say which; the reading taken
    is that consecutive groups of G value heads share a head: value head hv
    reads head hv // G.  Returns q and k widened to [B, T, Hv, d_k] so that
    ``recurrent`` / ``chunked_wy`` apply per value head unchanged.
    """
    q, k = _f64(q), _f64(k)
    H = q.shape[2]
    if k.shape != q.shape or Hv <= 0 or H <= 0 or Hv % H:
        raise ValueError(f"value heads {Hv} must be a positive multiple of query/key heads {H}")
    src = np.arange(Hv) // (Hv // H)          # the query/key head of each value head
    return q[:, :, src], k[:, :, src]


def varlen(cu_seqlens, q, k, v, alpha, b, w, S0=None, form=None):
    """Packed batch of variable-length sequences, fp64.

    The recurrence of the burn-gdn2 README ("Architecture") runs per sequence,
    and each sequence starts from its own state (an empty one when none is
    given, README "Quick start").  A packed batch lays N sequences back to
    back along the token axis: sequence i holds tokens
    cu_seqlens[i] .. cu_seqlens[i+1]-1 of the [1, T, H, *] tensors and
    starts from S0[i].  No state crosses a sequence boundary.

    cu_seqlens: N+1 nondecreasing offsets with cu_seqlens[0] = 0 and
    cu_seqlens[N] = T.  q, k: [1, T, H, d_k]; v, w: [1, T, H, d_v] (widen q, k
    with ``share_qk_heads`` first for grouped value heads); alpha, b:
    [1, T, H, d_k]; S0: [N, H, d_k, d_v] or None.  ``form`` is the per-batch
    function applied to each sequence (default ``recurrent``).
    Returns o [1, T, H, d_v] and S [N, H, d_k, d_v], fp64.
    """
    form = recurrent if form is None else form
    cu = [int(x) for x in np.asarray(cu_seqlens).ravel()]
    T = np.asarray(v).shape[1]
    if len(cu) < 1 or cu[0] != 0 or cu[-1] != T or any(b_ < a_ for a_, b_ in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must rise from 0 to T")
    if np.asarray(v).shape[0] != 1:
        raise ValueError("a packed batch has batch dimension 1")
    N = len(cu) - 1
    H, dk, dv = np.asarray(v).shape[2], np.asarray(alpha).shape[3], np.asarray(v).shape[3]
    o = np.zeros((1, T, H, dv))
    S = np.zeros((N, H, dk, dv))
    for i in range(N):
        s, e = cu[i], cu[i + 1]
        sl = lambda x: np.ascontiguousarray(np.asarray(x)[:, s:e])
        s0 = None if S0 is None else np.ascontiguousarray(np.asarray(S0)[i:i + 1])
        if e == s:          # an empty sequence leaves its state as it was
            S[i] = 0.0 if s0 is None else s0[0]
            continue
        oi, Si = form(sl(q), sl(k), sl(v), sl(alpha), sl(b), sl(w), s0)
        o[:, s:e] = oi
        S[i] = Si[0]
    return o, S


NORM_EPS = 1e-5   # burn-gdn2 README, "Configuration": norm_eps


def gated_rmsnorm(o, g, weight, eps=NORM_EPS):
    """The layer's output step after the core, fp64.

    burn-gdn2 README, "Architecture" diagram: the core's output goes through a
    gated RMS norm fed by a SiLU gate (the G projection), then the output
    projection; "Configuration" gives norm_eps = 1e-5.  Reading taken: per
    (token, head) over the d_v channels,

        y = o / sqrt(mean(o^2) + eps) * weight * silu(g),   silu(x) = x * sigmoid(x),

    with one weight vector of length d_v shared by all heads.

    o, g: [..., d_v]; weight: [d_v].  Returns fp64 y of o's shape.
    """
    o, g, weight = _f64(o), _f64(g), _f64(weight)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / rms * weight * (g * sigmoid(g))


CONV_SILU = 1   # the library's GDN2_CONV_SILU


def short_conv(x, weight, state=None, silu=False):
    """The layer's short convolution before the core, fp64.

    burn-gdn2 README, "Architecture" diagram: the projections go through a
    ShortConv before the L2 norm; "Configuration": use_short_conv = true, a
    depthwise convolution before the recurrence.  Its width and activation
    are not on the page.  Reading taken: a causal depthwise convolution over
    the token axis, one filter of K taps per channel,

        z[t, c] = sum_{i=0}^{K-1} weight[c, i] * x[t - (K-1) + i, c],

    y = z, or z * sigmoid(z) with the SiLU option.  Positions before the
    first token are read from `state`, the last K-1 inputs before it (oldest
    first; zeros when None), so that a sequence can be processed in pieces.

    x: [B, T, C]; weight: [C, K]; state: [B, K-1, C] or None.
    Returns fp64 y [B, T, C] and the state after the last token [B, K-1, C].
    """
    x, weight = _f64(x), _f64(weight)
    B, T, C = x.shape
    K = weight.shape[1]
    st = np.zeros((B, K - 1, C)) if state is None else _f64(state)
    xe = np.concatenate([st, x], axis=1)          # window: x at t - (K-1) + i is xe[t + i]
    z = np.zeros((B, T, C))
    for i in range(K):
        z += weight[:, i] * xe[:, i:i + T, :]
    y = z * sigmoid(z) if silu else z
    return y, xe[:, T:, :]


def short_conv_bwd(x, weight, dy, state=None, silu=False, dstate_out=None):
    """Gradients of sum(dy * y) + sum(dstate_out * state_out), where
    (y, state_out) = short_conv(x, weight, state, silu), fp64.

    With z the pre-activation and dz = dy (or dy * d silu/dz = dy * s (1 + z (1 - s)),
    s = sigmoid(z)), every input of the window xe = [state, x] receives
        d xe[p] = sum_i weight[:, i] * dz[p - i]      (dz = 0 outside [0, T)),
    and every tap  d weight[c, i] = sum over b, t of dz[b, t, c] * xe[b, t + i, c].
    state_out is the last K-1 entries of xe, so dstate_out (None = zeros) is
    added to d xe there: the gradient a following piece's backward hands back
    when a sequence is processed in pieces.
    Returns dx [B, T, C], dweight [C, K], dstate [B, K-1, C].
    """
    x, weight, dy = _f64(x), _f64(weight), _f64(dy)
    B, T, C = x.shape
    K = weight.shape[1]
    st = np.zeros((B, K - 1, C)) if state is None else _f64(state)
    xe = np.concatenate([st, x], axis=1)
    z = np.zeros((B, T, C))
    for i in range(K):
        z += weight[:, i] * xe[:, i:i + T, :]
    if silu:
        s = sigmoid(z)
        dz = dy * s * (1.0 + z * (1.0 - s))
    else:
        dz = dy
    dxe = np.zeros_like(xe)
    dw = np.zeros((C, K))
    for i in range(K):
        dxe[:, i:i + T, :] += weight[:, i] * dz
        dw[:, i] = np.sum(dz * xe[:, i:i + T, :], axis=(0, 1))
    if dstate_out is not None:
        dxe[:, T:, :] += _f64(dstate_out)
    return dxe[:, K - 1:, :], dw, dxe[:, :K - 1, :]


def recurrent(q, k, v, alpha, b, w, S0=None):
    """Sequential fp64 recurrence, literal order of the README's formula.

    burn-gdn2 README, "Architecture": per token, the state is decayed on the
    key axis (diag(alpha_t)), multiplied by the erase matrix
    E_t = I - k_t (b_t*k_t)^T, and receives the write k_t (w_t*v_t)^T; the
    output is q_t^T applied to the updated state.

    The erase matrix is formed explicitly (a d_k x d_k matrix per head and
    token) so that the code reads as the formula; this is O(d_k^2 d_v) per
    token and meant for small shapes.  Returns (o, S_T) in fp64.
    """
    q, k, v, alpha, b, w = map(_f64, (q, k, v, alpha, b, w))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, T, H, dv))
    eye = np.eye(dk)
    for t in range(T):
        kt = k[:, t]                                   # [B,H,dk]
        E = eye - kt[..., :, None] * (b[:, t] * kt)[..., None, :]   # I - k (b*k)^T
        D = alpha[:, t][..., :, None] * eye            # diag(alpha_t)
        write = kt[..., :, None] * (w[:, t] * v[:, t])[..., None, :]  # k (w*v)^T
        S = E @ (D @ S) + write
        o[:, t] = np.einsum("bhc,bhcj->bhj", q[:, t], S)   # q_t^T S_t
    return o, S


def chunked_wy(q, k, v, alpha, b, w, S0=None, chunk=64, return_intermediates=False):
    """fp64 chunked form of the same recurrence (chunk size ``chunk``).

    The README (intro and "Architecture" diagram; "Configuration" gives
    chunk_size = 64) names a chunked WY decomposition as the training-mode
    forward.  The pages give no formulas for it, so this is the form that the
    per-token recurrence itself implies, written per chunk of L tokens that
    enters with state S0 (positions r, s = 1..L inside the chunk):

      g_r = log alpha_r, G_r = sum_{j<=r} g_j, Gamma_r = exp(G_r)   (per key channel)
      e_r = b_r * k_r,   u_r = w_r * v_r
      A[r,s] = sum_c e_r[c] k_s[c] exp(G_r[c]-G_s[c])     for s <  r  (else 0)
      P[r,s] = sum_c q_r[c] k_s[c] exp(G_r[c]-G_s[c])     for s <= r  (else 0)
      Tm = (I + A)^{-1}
      W  = Tm @ (Gamma * e),   U = Tm @ u
      Delta = U - W @ S0
      O     = (Gamma * q) @ S0 + P @ Delta
      S_L   = diag(Gamma_L) @ S0 + Ktil^T @ Delta,   Ktil_s = k_s * exp(G_L - G_s)

    Derivation: one step is S_r = D_r S_{r-1} + k_r delta_r^T with
    delta_r = u_r - S_{r-1}^T (alpha_r * e_r); unrolling S_{r-1} and collecting
    the delta terms gives (I + A) Delta = U - (Gamma*e) S0.  A trailing partial
    chunk is handled at its own length.

    Returns (o, S_T); with ``return_intermediates`` also a list (one dict per
    (chunk, b, h) in that nesting order) holding G, A, P, Tm, W, U, Qh, Ktil,
    GammaL for kernel-level checks.
    """
    q, k, v, alpha, b, w = map(_f64, (q, k, v, alpha, b, w))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, T, H, dv))
    inter = []
    for n0 in range(0, T, chunk):
        L = min(chunk, T - n0)
        sl = slice(n0, n0 + L)
        for bi in range(B):
            for hi in range(H):
                qc = q[bi, sl, hi]          # [L,dk]
                kc = k[bi, sl, hi]
                ec = b[bi, sl, hi] * kc
                uc = w[bi, sl, hi] * v[bi, sl, hi]   # [L,dv]
                G = np.cumsum(np.log(alpha[bi, sl, hi]), axis=0)   # [L,dk]
                ratio = np.exp(G[:, None, :] - G[None, :, :])       # [r,s,c]
                A = np.einsum("rc,sc,rsc->rs", ec, kc, ratio) * np.tri(L, k=-1)
                P = np.einsum("rc,sc,rsc->rs", qc, kc, ratio) * np.tri(L, k=0)
                Tm = np.linalg.inv(np.eye(L) + A)
                Gam = np.exp(G)
                W = Tm @ (Gam * ec)
                U = Tm @ uc
                S0c = S[bi, hi]
                Delta = U - W @ S0c
                Qh = Gam * qc
                o[bi, sl, hi] = Qh @ S0c + P @ Delta
                Ktil = kc * np.exp(G[-1][None, :] - G)
                S[bi, hi] = Gam[-1][:, None] * S0c + Ktil.T @ Delta
                if return_intermediates:
                    inter.append(dict(G=G, A=A, P=P, Tm=Tm, W=W, U=U, Qh=Qh,
                                      Ktil=Ktil, GammaL=Gam[-1]))
    if return_intermediates:
        return o, S, inter
    return o, S


def rel_l2(x, ref):
    """||x - ref||_2 / ||ref||_2 over the whole tensor in fp64 (max-abs if ref == 0)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"rel_l2: shapes differ, {x.shape} vs {ref.shape}")
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return float(np.max(np.abs(x - ref))) if x.size else 0.0
    return float(num / den)


def rel_l2_chains(x, ref, chain_axes):
    """rel_l2 of every chain: the sub-tensors indexed by ``chain_axes`` (e.g. (0, 2) for
    o [B,T,H,dv], (0, 1) for S [B,H,dk,dv]), each over all its other elements.  Returns
    an array shaped like those axes."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"rel_l2_chains: shapes differ, {x.shape} vs {ref.shape}")
    rest = [a for a in range(x.ndim) if a not in chain_axes]
    xs = np.transpose(x, list(chain_axes) + rest)
    rs = np.transpose(ref, list(chain_axes) + rest)
    lead = xs.shape[:len(chain_axes)]
    xs = xs.reshape(lead + (-1,))
    rs = rs.reshape(lead + (-1,))
    out = np.zeros(lead)
    for idx in np.ndindex(*lead):
        out[idx] = rel_l2(xs[idx], rs[idx])
    return out
