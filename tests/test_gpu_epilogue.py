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
    """The chunked workload's o (B4 H16 T2048 dv128), sampled rows against the oracle."""
    o, gt, wt = _draw(dev, (4, 2048, 16, 128), torch.bfloat16, seed=5)
    y = g.gated_rmsnorm(o, gt, wt)
    torch.cuda.synchronize()
    idx = (np.array([0, 1, 3]), np.array([0, 1000, 2047]), np.array([0, 7, 15]))
    ref = gated_rmsnorm(_np(o)[idx], _np(gt)[idx], _np(wt))
    assert rel_l2(_np(y)[idx], ref) <= 2e-2
