"""GPU parity of the output step, the gated RMS norm, against the fp64 oracle (needs an MI355X).

y = o / sqrt(mean(o^2) + 1e-5) * weight * silu(g) per (token, head) row
(burn-gdn2 README "Architecture" / "Configuration").  Both sides get the same
seeded o, g (bf16 widened exactly) and weight; rel-L2 <= 1e-4 with fp32 I/O,
<= 2e-2 with bf16 (the output is rounded to bf16 once).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as g
from oracle.reference import gated_rmsnorm, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()
    return torch.device("cuda:0")


def _np(x):
    return x.detach().to("cpu", torch.float32).numpy()


def _draw(dev, shape, dt, seed):
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    o = (torch.randn(*shape, generator=gen, device=dev) * 0.7).to(dt)
    gt = torch.randn(*shape, generator=gen, device=dev).to(dt)
    wt = torch.randn(shape[-1], generator=gen, device=dev) * 0.5 + 1.0
    return o, gt, wt


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(1, 5, 2, 16), (2, 37, 3, 48), (2, 100, 4, 128), (1, 33, 2, 256),
                                   (3, 7, 1, 80)])
def test_gated_rmsnorm(dev, shape, dt):
    o, gt, wt = _draw(dev, shape, dt, seed=sum(shape))
    y = g.gated_rmsnorm(o, gt, wt)
    torch.cuda.synchronize()
    ref = gated_rmsnorm(_np(o), _np(gt), _np(wt))
    e = rel_l2(_np(y), ref)
    tol = 1e-4 if dt == torch.float32 else 2e-2
    print(f"[parity] gated_rmsnorm {shape} {dt}: relL2 {e:.3e}", flush=True)
    assert e <= tol


def test_gated_rmsnorm_in_place_after_the_chunked_forward(dev):
    """o of a chunked forward, normalised in place, equals the out-of-place result bit for bit."""
    from gated_delta_rule_19_amd import inputs
    inp = inputs.make_raw(2, 150, 4, 128, 128, torch.bfloat16, 9, dev)
    o, _ = g.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"])
    gt = torch.randn_like(o.float()).to(torch.bfloat16)
    wt = torch.ones(128, device=dev)
    y = g.gated_rmsnorm(o, gt, wt)
    g.gated_rmsnorm(o, gt, wt, inplace=True)
    torch.cuda.synchronize()
    assert torch.equal(y, o)


def test_gated_rmsnorm_full_chunk_size(dev):
    """The chunked workload's o (B4 H16 T2048 dv128): the whole tensor against the oracle,
    and the worst (token, head) row held to the same bar."""
    o, gt, wt = _draw(dev, (4, 2048, 16, 128), torch.bfloat16, seed=5)
    y = g.gated_rmsnorm(o, gt, wt)
    torch.cuda.synchronize()
    ref = gated_rmsnorm(_np(o), _np(gt), _np(wt))
    yn = _np(y).astype(np.float64)
    e = rel_l2(yn, ref)
    rows = np.linalg.norm((yn - ref).reshape(-1, 128), axis=1) / np.linalg.norm(ref.reshape(-1, 128), axis=1)
    print(f"[parity] gated_rmsnorm B4 H16 T2048: relL2 {e:.3e}, worst row {rows.max():.3e}", flush=True)
    assert e <= 2e-2 and rows.max() <= 2e-2


# ---- the output step fused into the recurrent forward -----------------------------
GATED = [
    # B, T, H, Hv, dk, dv, io dtype, flags
    (256, 1, 16, 16, 128, 128, torch.bfloat16, 0),     # the decode workload's shape
    (8, 1, 4, 8, 128, 256, torch.bfloat16, 0),
    (4, 1, 2, 2, 64, 64, torch.float32, 0),
    (2, 37, 2, 4, 128, 128, torch.bfloat16, 7),        # several tokens, prologue flags, grouped heads
    (3, 5, 2, 2, 32, 32, torch.float32, 1),
    (2, 9, 1, 1, 16, 16, torch.bfloat16, 4),
]


@pytest.mark.parametrize("case", GATED, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}Hv{c[3]}dk{c[4]}dv{c[5]}"
                         f"{'bf16' if c[6] == torch.bfloat16 else 'f32'}fl{c[7]}")
def test_recurrent_with_output_step(dev, case):
    """gdn2_recurrent_step_gated against the oracle chain gated_rmsnorm(recurrent(...)) (the output
    step taken on the fp64 o), and the state against the plain recurrence; both modes' state updated
    in place."""
    from gated_delta_rule_19_amd import inputs
    from oracle import c_oracle
    from oracle.reference import share_qk_heads
    B, T, H, Hv, dk, dv, dt, fl = case
    inp = inputs.make_raw(B, T, H, dk, dv, dt, B + T + dv + fl, dev, s0_std=0.05, Hv=Hv,
                          gate_logits=bool(fl & 1), unit_qk=not fl & 4)
    gen = torch.Generator(device=dev)
    gen.manual_seed(B * T + dv)
    gt = torch.randn(inp["v"].shape, generator=gen, device=dev).to(dt)
    wt = torch.randn(dv, generator=gen, device=dev) * 0.5 + 1.0
    a = (inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"])
    h = {k_: (None if v_ is None else _np(v_)) for k_, v_ in inp.items()}
    qw, kw = share_qk_heads(h["q"], h["k"], Hv)
    ro, rS = c_oracle.recurrent(qw, kw, h["v"], h["alpha"], h["b"], h["w"], h["S0"], flags=fl)
    ry = gated_rmsnorm(ro, _np(gt), _np(wt))
    S = inp["S0"].clone()
    y, _ = g.recurrent_step_gated(*a, gt, wt, S, inplace=True, flags=fl)
    torch.cuda.synchronize()
    tol = 1e-4 if dt == torch.float32 else 2e-2
    ey, eS = rel_l2(_np(y), ry), rel_l2(_np(S), rS)
    print(f"[parity] recurrent + output step {case}: relL2 y={ey:.3e} S={eS:.3e}", flush=True)
    assert ey <= tol and eS <= tol
    # the state equals the plain recurrent step's up to the order of its fp32 sums (whole-row
    # workgroups here, slices there); y equals the separate output step within one rounding of o
    S2 = inp["S0"].clone()
    o2, _ = g.recurrent_step(*a, S2, inplace=True, flags=fl)
    y2 = g.gated_rmsnorm(o2, gt, wt)
    torch.cuda.synchronize()
    assert rel_l2(_np(S), _np(S2)) <= 1e-5
    assert rel_l2(_np(y), _np(y2)) <= (1e-5 if dt == torch.float32 else 1e-2)
