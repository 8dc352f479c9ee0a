"""Seeded synthetic inputs for the GDN-2 token mixer (shared by tests, bench, smoke).

This module holds only random-number generation and shape bookkeeping; none
of the token mixer's arithmetic lives here, so both the GPU path and the CPU
oracle can consume what it draws.

Recipe (per workload; draw order q, k, v, alpha-logits, b-logits, w-logits, S0):
  q, k ~ N(0, 1), each (batch, token, head) row L2-normalised along d_k in fp32
         (the layer normalises q and k before the core -- burn-gdn2 README,
         "Architecture" diagram -- so the core receives unit-norm rows), then
         rounded to the I/O dtype (RNE);
  v    ~ N(0, 1) rounded to the I/O dtype;
  alpha = sigmoid(N(alpha_mu, 1)) per key channel, fp32;
  b     = b_scale * sigmoid(N(0, 1)) per key channel, fp32 (b_scale = 2 is the
          README's negative-eigenvalue option, "b x 2");
  w     = sigmoid(N(0, 1)) per value channel, fp32;
  S0    = N(0, s0_std) fp32 when s0_std is given, else no initial state.

Prologue variants (for the kernels' in-kernel prologue options):
  gate_logits=True returns the gates' pre-activation draws instead of their
  sigmoids (alpha-logit ~ N(alpha_mu, 1), b-logit ~ N(0, 1), w-logit ~ N(0, 1);
  b_scale is then the kernels' job), unit_qk=False leaves q and k unnormalised
  (N(0, 1) rows), and gate_dtype sets the gates' dtype (rounded RNE).

Grouped value heads: Hv (default H) value heads, a multiple of H; q and k are
drawn for the H query/key heads, v, the gates and S0 for the Hv value heads.

Packed variable-length batches (``make_packed``): the token tensors of one
[1, T, *, *] batch with T = sum of the lengths, drawn as above, plus one
initial state per sequence and the int32 offsets cu_seqlens.  The length mix
(``length_mix``) draws log-uniform lengths in [lo, hi] until the total is
reached (the last one cut to fit).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    io_dtype: torch.dtype
    alpha_mu: float = 3.0
    b_scale: float = 1.0
    s0_std: Optional[float] = None
    mode: str = "chunk"          # "chunk" | "recurrent" | "decode"
    note: str = field(default="", compare=False)

    @property
    def head_tokens(self) -> int:
        return self.B * self.T * self.H


# The five synthetic workloads the path is built and measured on.
WORKLOADS = {
    0: Workload("tiny-fp32", 1, 64, 2, 16, 16, torch.float32, mode="both",
                note="oracle-size check of both modes, fp32 I/O"),
    1: Workload("chunk-B4-H16-T2048-d128", 4, 2048, 16, 128, 128, torch.bfloat16,
                note="chunked forward at a 1.3B-layer shape (hidden 2048)"),
    2: Workload("decode-B256-H16-d128", 256, 1, 16, 128, 128, torch.bfloat16,
                s0_std=0.05, mode="decode",
                note="one fused recurrent decode step, fp32 state updated in place"),
    3: Workload("chunk-B1-H16-T65536-d128", 1, 65536, 16, 128, 128, torch.bfloat16,
                alpha_mu=4.0, note="long-context chunked forward, slow decay"),
    4: Workload("chunk-B8-H16-T4096-dk128-dv256", 8, 4096, 16, 128, 256, torch.bfloat16,
                b_scale=2.0, s0_std=0.05,
                note="expanded values, b in (0,2), nonzero initial state"),
}


def make(wl: Workload, seed: int, device="cpu", B=None, T=None, H=None):
    """Draw one input set for ``wl`` (optionally overriding B/T/H).

    Returns a dict with q, k, v (io dtype), alpha, b, w (fp32), S0 (fp32 or None).
    """
    B = wl.B if B is None else B
    T = wl.T if T is None else T
    H = wl.H if H is None else H
    return make_raw(B, T, H, wl.dk, wl.dv, wl.io_dtype, seed, device,
                    alpha_mu=wl.alpha_mu, b_scale=wl.b_scale, s0_std=wl.s0_std)


def make_raw(B, T, H, dk, dv, io_dtype, seed, device="cpu", alpha_mu=3.0,
             b_scale=1.0, s0_std=None, gate_logits=False, unit_qk=True, gate_dtype=torch.float32, Hv=None,
             n_states=None):
    """One input set; ``n_states`` initial states (default B) when ``s0_std`` is given."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    f32 = torch.float32

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=dev, dtype=f32)

    def unit_rows(x):
        n = torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x / torch.clamp(n, min=1e-30)

    rows = unit_rows if unit_qk else (lambda x: x)
    Hv = H if Hv is None else Hv
    q = rows(randn(B, T, H, dk)).to(io_dtype)
    k = rows(randn(B, T, H, dk)).to(io_dtype)
    v = randn(B, T, Hv, dv).to(io_dtype)
    la, lb, lw = randn(B, T, Hv, dk) + alpha_mu, randn(B, T, Hv, dk), randn(B, T, Hv, dv)
    if gate_logits:
        alpha, b, w = la, lb, lw
    else:
        alpha, b, w = torch.sigmoid(la), b_scale * torch.sigmoid(lb), torch.sigmoid(lw)
    alpha, b, w = alpha.to(gate_dtype), b.to(gate_dtype), w.to(gate_dtype)
    S0 = None
    if s0_std is not None:
        S0 = randn(B if n_states is None else n_states, Hv, dk, dv) * s0_std
    return dict(q=q, k=k, v=v, alpha=alpha, b=b, w=w, S0=S0)


def make_out_grads(B, T, H, dk, dv, io_dtype, seed, device="cpu", state_grad=True):
    """Seeded output gradients for the backward: dO ~ N(0, 1) [B,T,H,dv] in the I/O dtype,
    dS_T ~ N(0, 1) [B,H,dk,dv] fp32 (None without ``state_grad``)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    dO = torch.randn(B, T, H, dv, generator=g, device=dev).to(io_dtype)
    dS = torch.randn(B, H, dk, dv, generator=g, device=dev) if state_grad else None
    return dO, dS


def length_mix(total, seed, lo=16, hi=4096):
    """Seeded sequence lengths summing to ``total``: log-uniform in [lo, hi], last one cut."""
    g = torch.Generator()
    g.manual_seed(int(seed))
    out, left = [], int(total)
    while left > 0:
        u = torch.rand((), generator=g).item()
        n = int(round(lo * (hi / lo) ** u))
        n = max(1, min(n, left))
        out.append(n)
        left -= n
    return out


def make_packed(lengths, H, dk, dv, io_dtype, seed, device="cpu", **kw):
    """A packed batch of len(lengths) sequences: make_raw's tensors for [1, sum(lengths)],
    S0 per sequence (with ``s0_std``), and ``cu`` = int32 offsets [N+1] on ``device``."""
    T = int(sum(lengths))
    inp = make_raw(1, T, H, dk, dv, io_dtype, seed, device, n_states=len(lengths), **kw)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    inp["cu"] = torch.tensor(cu, dtype=torch.int32, device=torch.device(device))
    return inp


def to_numpy_f32(inp):
    """Exact float32 widening of every tensor (bf16 -> fp32 is exact), on the host."""
    out = {}
    for key, x in inp.items():
        out[key] = None if x is None else x.detach().to("cpu", torch.float32).numpy()
    return out
