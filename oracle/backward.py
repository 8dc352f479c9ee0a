"""fp64 CPU oracle of the GDN-2 backward pass (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU leg may
import this module; the GPU library shares no code with it.

The forward is the per-token recurrence of the burn-gdn2 0.1.9 README,
section "Architecture"; the README calls the chunked WY mode the training
mode but prints no gradient.  The gradient of a function is unique, so both
routines below compute the same thing: the derivative of

    loss = sum(dO * o) + sum(dS_T * S_T)

with respect to every input (q, k, v, alpha, b, w, S0), for given output
gradients dO [B,T,H,dv] and dS_T [B,H,dk,dv] (None = 0).  Layouts as in
``oracle.reference``.  Both are pinned against central finite differences.

``recurrent_bwd`` reverses the recurrence token by token.  With
z_t = alpha_t * b_t * k_t and u_t = w_t * v_t one step reads

    S_t = diag(alpha_t) S_{t-1} + k_t delta_t^T,   delta_t = u_t - S_{t-1}^T z_t,

so, with G_t the gradient of S_t (from o_t = S_t^T q_t and from S_{t+1}):

    G_t      += q_t dO_t^T                 dq_t = S_t dO_t
    ddelta_t  = G_t^T k_t                  dk_t = G_t delta_t + (dz_t * alpha_t * b_t)
    du_t      = ddelta_t                   dw_t = du_t * v_t,  dv_t = du_t * w_t
    dz_t      = -S_{t-1} ddelta_t          db_t = dz_t * alpha_t * k_t
    dalpha_t  = rowsum(G_t * S_{t-1}) + dz_t * b_t * k_t
    G_{t-1}   = diag(alpha_t) G_t - z_t ddelta_t^T          (dS0 = G_0)

``chunked_bwd`` is the chunk-level form the GPU kernels follow (chunk length
C, positions r, s inside a chunk, the forward's notation of
``oracle.reference.chunked_wy``):
  1. forward over chunks, keeping the state S_n entering each chunk;
  2. backward over chunks from dS = dS_T: the gradient leaving chunk n is
     dSL_n = dS; then
        dDelta = P^T dO + Ktil dSL
        dS     = Qh^T dO + diag(Gamma_L) dSL - W^T dDelta
     and dS0 is the dS left after chunk 0;
  3. per chunk, from S0 = S_n, dSL = dSL_n and dO:
        Delta = U - W S0
        dQh = dO S0^T,  dP = mask_{s<=r}(dO Delta^T),  dKtil = Delta dSL^T,
        dGammaL = rowsum(dSL * S0),  dW = -dDelta S0^T,  du = Tm^T dDelta,
        dTm = dDelta u^T + dW Eh^T,  dEh = Tm^T dW,
        dA  = mask_{s<r}(-Tm^T dTm Tm^T)
     and through the definitions of Qh = Gamma*q, Eh = Gamma*e, Ktil, A, P:
        dq  = Gamma*dQh + sum_s dP[r,s] k_s R[r,s]
        de  = Gamma*dEh + sum_s dA[r,s] k_s R[r,s]
        dk  = exp(G_L - G)*dKtil + sum_r (dA[r,s] e_r + dP[r,s] q_r) R[r,s] + de*b
        dG_r = dQh*Qh + dEh*Eh - dKtil*Ktil + sum_s (dA e_r k_s + dP q_r k_s) R[r,s]
                                            - sum_r' (dA[r',r] e_r' k_r + dP[r',r] q_r' k_r) R[r',r]
        dG_L += sum_s dKtil_s*Ktil_s + dGammaL*Gamma_L
     (R[r,s] = exp(G_r - G_s) per key channel); then dlog(alpha) is the
     reverse cumulative sum of dG inside the chunk, dalpha = dlog(alpha)/alpha,
     db = de*k, du = dw/v-style split as above.
"""
from __future__ import annotations

import numpy as np

from .reference import _f64

__all__ = ["recurrent_bwd", "chunked_bwd", "full_bwd", "loss"]


def loss(o, S, dO, dS_T=None):
    """The scalar whose gradient both routines return."""
    val = float(np.sum(_f64(o) * _f64(dO)))
    if dS_T is not None:
        val += float(np.sum(_f64(S) * _f64(dS_T)))
    return val


def _states(q, k, v, alpha, b, w, S0):
    """Forward recurrence keeping every state: returns S[t] for t = -1..T-1 as an array
    of T+1 states per (batch, head) ([T+1, B, H, dk, dv]) and o."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else S0.copy()
    out = [S.copy()]
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        z = alpha[:, t] * b[:, t] * k[:, t]
        u = w[:, t] * v[:, t]
        delta = u - np.einsum("bhcj,bhc->bhj", S, z)
        S = alpha[:, t][..., None] * S + k[:, t][..., :, None] * delta[..., None, :]
        o[:, t] = np.einsum("bhc,bhcj->bhj", q[:, t], S)
        out.append(S.copy())
    return np.stack(out), o


def recurrent_bwd(q, k, v, alpha, b, w, S0, dO, dS_T=None):
    """Token-by-token reverse of the recurrence (see the module docstring).
    Returns dict dq, dk, dv, dalpha, db, dw, dS0 (fp64)."""
    q, k, v, alpha, b, w, dO = map(_f64, (q, k, v, alpha, b, w, dO))
    S0 = None if S0 is None else _f64(S0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    Ss, _ = _states(q, k, v, alpha, b, w, S0)
    G = np.zeros((B, H, dk, dv)) if dS_T is None else _f64(dS_T).copy()
    g = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha), ("db", b),
                                          ("dw", w))}
    for t in range(T - 1, -1, -1):
        St, Sp = Ss[t + 1], Ss[t]
        G = G + q[:, t][..., :, None] * dO[:, t][..., None, :]
        g["dq"][:, t] = np.einsum("bhcj,bhj->bhc", St, dO[:, t])
        z = alpha[:, t] * b[:, t] * k[:, t]
        u = w[:, t] * v[:, t]
        delta = u - np.einsum("bhcj,bhc->bhj", Sp, z)
        ddelta = np.einsum("bhcj,bhc->bhj", G, k[:, t])
        dz = -np.einsum("bhcj,bhj->bhc", Sp, ddelta)
        g["dk"][:, t] = np.einsum("bhcj,bhj->bhc", G, delta) + dz * alpha[:, t] * b[:, t]
        g["dw"][:, t] = ddelta * v[:, t]
        g["dv"][:, t] = ddelta * w[:, t]
        g["db"][:, t] = dz * alpha[:, t] * k[:, t]
        g["dalpha"][:, t] = np.sum(G * Sp, axis=-1) + dz * b[:, t] * k[:, t]
        G = alpha[:, t][..., None] * G - z[..., :, None] * ddelta[..., None, :]
    g["dS0"] = G
    return g


def _chunk_factors(qc, kc, bc, ac, uc):
    """Forward factors of one chunk (positions 0..L-1), fp64."""
    L = qc.shape[0]
    ec = bc * kc
    G = np.cumsum(np.log(ac), axis=0)
    R = np.exp(G[:, None, :] - G[None, :, :])            # [r, s, c]
    A = np.einsum("rc,sc,rsc->rs", ec, kc, R) * np.tri(L, k=-1)
    P = np.einsum("rc,sc,rsc->rs", qc, kc, R) * np.tri(L, k=0)
    Tm = np.linalg.inv(np.eye(L) + A)
    Gam = np.exp(G)
    Eh = Gam * ec
    Ktil = kc * np.exp(G[-1][None, :] - G)
    return dict(e=ec, G=G, R=R, A=A, P=P, Tm=Tm, Gam=Gam, Eh=Eh, Qh=Gam * qc, Ktil=Ktil,
                W=Tm @ Eh, U=Tm @ uc)


def chunked_bwd(q, k, v, alpha, b, w, S0, dO, dS_T=None, chunk=64):
    """Chunk-level backward in the steps the GPU follows (see the module docstring).
    Returns the same dict as ``recurrent_bwd``."""
    q, k, v, alpha, b, w, dO = map(_f64, (q, k, v, alpha, b, w, dO))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    g = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha), ("db", b),
                                          ("dw", w))}
    g["dS0"] = np.zeros((B, H, dk, dv))
    starts = list(range(0, T, chunk))
    for bi in range(B):
        for hi in range(H):
            # 1. forward over chunks, keeping each chunk's entering state
            S = np.zeros((dk, dv)) if S0 is None else _f64(S0)[bi, hi].copy()
            fac, Sn = [], []
            for n0 in starts:
                sl = slice(n0, min(n0 + chunk, T))
                f = _chunk_factors(q[bi, sl, hi], k[bi, sl, hi], b[bi, sl, hi], alpha[bi, sl, hi],
                                   w[bi, sl, hi] * v[bi, sl, hi])
                Sn.append(S.copy())
                Delta = f["U"] - f["W"] @ S
                S = f["Gam"][-1][:, None] * S + f["Ktil"].T @ Delta
                fac.append(f)
            # 2. backward over chunks: the gradient leaving each chunk
            dS = np.zeros((dk, dv)) if dS_T is None else _f64(dS_T)[bi, hi].copy()
            dSL = [None] * len(starts)
            for n in range(len(starts) - 1, -1, -1):
                f = fac[n]
                dOc = dO[bi, starts[n]:starts[n] + f["P"].shape[0], hi]
                dSL[n] = dS.copy()
                dDelta = f["P"].T @ dOc + f["Ktil"] @ dS
                dS = f["Qh"].T @ dOc + f["Gam"][-1][:, None] * dS - f["W"].T @ dDelta
            g["dS0"][bi, hi] = dS
            # 3. per-chunk gradients
            for n, n0 in enumerate(starts):
                f = fac[n]
                L = f["P"].shape[0]
                sl = slice(n0, n0 + L)
                qc, kc, bc, ac = q[bi, sl, hi], k[bi, sl, hi], b[bi, sl, hi], alpha[bi, sl, hi]
                vc, wc = v[bi, sl, hi], w[bi, sl, hi]
                uc = wc * vc
                dOc = dO[bi, sl, hi]
                S0c, dSLc = Sn[n], dSL[n]
                Tm, R, e = f["Tm"], f["R"], f["e"]
                Delta = f["U"] - f["W"] @ S0c
                dDelta = f["P"].T @ dOc + f["Ktil"] @ dSLc
                dQh = dOc @ S0c.T
                dP = (dOc @ Delta.T) * np.tri(L, k=0)
                dKtil = Delta @ dSLc.T
                dGamL = np.sum(dSLc * S0c, axis=1)
                dW = -dDelta @ S0c.T
                du = Tm.T @ dDelta
                dTm = dDelta @ uc.T + dW @ f["Eh"].T
                dEh = Tm.T @ dW
                dA = (-Tm.T @ dTm @ Tm.T) * np.tri(L, k=-1)
                # through Qh, Eh, Ktil, A, P
                dq = f["Gam"] * dQh + np.einsum("rs,sc,rsc->rc", dP, kc, R)
                de = f["Gam"] * dEh + np.einsum("rs,sc,rsc->rc", dA, kc, R)
                dk = (np.exp(f["G"][-1][None, :] - f["G"]) * dKtil
                      + np.einsum("rs,rc,rsc->sc", dA, e, R) + np.einsum("rs,rc,rsc->sc", dP, qc, R))
                pair = (dA[:, :, None] * e[:, None, :] + dP[:, :, None] * qc[:, None, :]) * kc[None, :, :] * R
                dG = dQh * f["Qh"] + dEh * f["Eh"] - dKtil * f["Ktil"] + pair.sum(axis=1) - pair.sum(axis=0)
                dG[-1] += np.sum(dKtil * f["Ktil"], axis=0) + dGamL * f["Gam"][-1]
                dlog = np.cumsum(dG[::-1], axis=0)[::-1]
                g["dq"][bi, sl, hi] = dq
                g["dk"][bi, sl, hi] = dk + de * bc
                g["db"][bi, sl, hi] = de * kc
                g["dalpha"][bi, sl, hi] = dlog / ac
                g["dw"][bi, sl, hi] = du * vc
                g["dv"][bi, sl, hi] = du * wc
    return g


def full_bwd(q, k, v, alpha, b, w, S0, dO, dS_T=None, flags=0):
    """Gradients with the prologue options and grouped value heads, fp64.

    The forward is: the prologue (``oracle.reference.prologue``: sigmoid of gate
    logits, b x 2, q/k L2 norm), then, with more value heads than query/key
    heads, the query/key heads shared by consecutive groups of value heads
    (``oracle.reference.share_qk_heads``), then the recurrence.  The gradient
    runs back through the three steps:
      * ``recurrent_bwd`` on the activated, widened inputs;
      * each query/key head gets the sum of its group's dq and dk;
      * L2 norm: with n = sqrt(sum(x^2) + eps) and xh = x / n,
        dx = (dxh - xh * sum(xh * dxh)) / n per (token, head);
      * logits: dlogit = dgate * s (1 - s) with s = sigmoid(logit), times 2
        for b in negative-eigenvalue mode.
    q, k: [B, T, H, dk]; v, w: [B, T, Hv, dv]; alpha, b: [B, T, Hv, dk].
    """
    from .reference import FLAG_GATE_LOGITS, FLAG_NEG_EIGVAL, FLAG_QK_L2NORM, L2NORM_EPS, prologue, \
        share_qk_heads, sigmoid
    q, k, v, alpha, b, w, dO = map(_f64, (q, k, v, alpha, b, w, dO))
    B, T, H, dk = q.shape
    Hv = v.shape[2]
    pq, pk, pa, pb, pw = prologue(q, k, alpha, b, w, flags)
    qg, kg = share_qk_heads(pq, pk, Hv) if Hv != H else (pq, pk)
    g = recurrent_bwd(qg, kg, v, pa, pb, pw, S0, dO, dS_T)
    G = Hv // H
    dq = g["dq"].reshape(B, T, H, G, dk).sum(axis=3)
    dk_ = g["dk"].reshape(B, T, H, G, dk).sum(axis=3)
    if flags & FLAG_QK_L2NORM:
        def back(x, dxh):
            n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2NORM_EPS)
            xh = x / n
            return (dxh - xh * np.sum(xh * dxh, axis=-1, keepdims=True)) / n
        dq, dk_ = back(q, dq), back(k, dk_)
    out = dict(dq=dq, dk=dk_, dv=g["dv"], dalpha=g["dalpha"], db=g["db"], dw=g["dw"], dS0=g["dS0"])
    if flags & FLAG_GATE_LOGITS:
        for name, x, scale in (("dalpha", alpha, 1.0), ("db", b, 2.0 if flags & FLAG_NEG_EIGVAL else 1.0),
                               ("dw", w, 1.0)):
            s = sigmoid(x)
            out[name] = out[name] * s * (1.0 - s) * scale
    return out
