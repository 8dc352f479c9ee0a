"""GPU parity of the HIP path against the fp64 CPU oracle (needs an MI355X).

Every comparison feeds both sides the same seeded inputs (bf16 inputs are
widened exactly for the oracle) and measures the relative L2 error over the
whole tensor, for o and for the final state separately:
    <= 1e-4 for fp32 I/O, <= 2e-2 for bf16 I/O with the fp32 state.
Full-size workloads are compared on every (batch, head) chain against the
fp64 C oracle, with the GPU run in exactly the launch configuration the
benchmark times; the worst chain's error is reported beside the global one
(and held to the same bar).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as g
from gated_delta_rule_19_amd import inputs
from oracle import c_oracle
from oracle.reference import chunked_wy, rel_l2, rel_l2_chains

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()          # a missing library is an error on a GPU host
    return torch.device("cuda:0")


def _np(x):
    return None if x is None else x.detach().to("cpu", torch.float32).numpy()


def oracle(inp, S0=None, chains=None):
    """fp64 oracle on all chains, or on a list of (b, h) chains -> (o, S) stacked per chain."""
    h = {key: _np(val) for key, val in inp.items()}
    S0n = _np(S0) if S0 is not None else (h.get("S0"))
    if chains is None:
        return c_oracle.recurrent(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], S0n)
    outs, states = [], []
    for bi, hi in chains:
        sl = lambda x: np.ascontiguousarray(x[bi:bi + 1, :, hi:hi + 1])
        s0 = None if S0n is None else np.ascontiguousarray(S0n[bi:bi + 1, hi:hi + 1])
        o, S = c_oracle.recurrent(sl(h["q"]), sl(h["k"]), sl(h["v"]), sl(h["alpha"]), sl(h["b"]),
                                  sl(h["w"]), s0)
        outs.append(o[0, :, 0])
        states.append(S[0, 0])
    return np.stack(outs), np.stack(states)


def pick(o, S, chains):
    on = _np(o)
    Sn = _np(S)
    return (np.stack([on[bi, :, hi] for bi, hi in chains]),
            np.stack([Sn[bi, hi] for bi, hi in chains]))


def check(what, o, S, ref_o, ref_S, tol, chain_axes=((0, 2), (0, 1))):
    """Whole-tensor rel-L2 of o and S, and the worst (batch, head) chain of each
    (o [B,T,H,dv] chains on axes 0, 2; S [B,H,dk,dv] on axes 0, 1; pass chain_axes=None
    for stacked per-chain arrays, whose chains are axis 0)."""
    on = _np(o) if torch.is_tensor(o) else o
    Sn = _np(S) if torch.is_tensor(S) else S
    eo, eS = rel_l2(on, ref_o), rel_l2(Sn, ref_S)
    ax_o, ax_S = chain_axes if chain_axes is not None else ((0,), (0,))
    wo = float(np.max(rel_l2_chains(on, ref_o, ax_o))) if on.size else 0.0
    wS = float(np.max(rel_l2_chains(Sn, ref_S, ax_S))) if Sn.size else 0.0
    print(f"[parity] {what}: relL2 o={eo:.3e} S={eS:.3e}; worst chain o={wo:.3e} S={wS:.3e} (tol {tol:g})",
          flush=True)
    assert eo <= tol, f"{what}: o rel-L2 {eo:.3e} > {tol}"
    assert eS <= tol, f"{what}: S rel-L2 {eS:.3e} > {tol}"
    assert wo <= tol, f"{what}: worst chain o rel-L2 {wo:.3e} > {tol}"
    assert wS <= tol, f"{what}: worst chain S rel-L2 {wS:.3e} > {tol}"


def make(dev, B, T, H, dk, dv, dt, seed, s0=None, b_scale=1.0, alpha_mu=3.0):
    return inputs.make_raw(B, T, H, dk, dv, dt, seed, dev, alpha_mu=alpha_mu, b_scale=b_scale,
                           s0_std=s0)


def args(inp):
    return inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"]


SMALL = [
    # B, T, H, dk, dv, dtype, S0 std, b scale
    (1, 64, 2, 16, 16, torch.float32, None, 1.0),      # tiny fp32 workload
    (2, 37, 3, 128, 128, torch.bfloat16, 0.05, 1.0),
    (1, 200, 2, 128, 128, torch.bfloat16, 0.05, 2.0),
    (1, 130, 2, 64, 48, torch.bfloat16, None, 1.0),
    (2, 70, 2, 32, 256, torch.float32, 0.05, 2.0),
    (1, 100, 2, 16, 32, torch.bfloat16, 0.05, 1.0),
    (1, 150, 3, 32, 48, torch.float32, None, 1.0),
    (1, 90, 1, 128, 256, torch.bfloat16, 0.05, 2.0),
    (2, 65, 2, 64, 64, torch.float32, 0.05, 1.0),
]


def _id(c):
    B, T, H, dk, dv, dt, s0, bs = c
    return f"B{B}T{T}H{H}dk{dk}dv{dv}{'bf16' if dt == torch.bfloat16 else 'f32'}{'S0' if s0 else ''}b{bs:g}"


@pytest.mark.parametrize("case", SMALL, ids=_id)
def test_recurrent_small(dev, case):
    B, T, H, dk, dv, dt, s0, bs = case
    inp = make(dev, B, T, H, dk, dv, dt, seed=T * 7 + dk, s0=s0, b_scale=bs)
    o, S = g.recurrent_step(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    ro, rS = oracle(inp)
    check("recurrent " + _id(case), o, S, ro, rS, TOL[dt])


@pytest.mark.parametrize("case", SMALL, ids=_id)
def test_chunk_small(dev, case):
    B, T, H, dk, dv, dt, s0, bs = case
    inp = make(dev, B, T, H, dk, dv, dt, seed=T * 11 + dv, s0=s0, b_scale=bs)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    ro, rS = oracle(inp)
    check("chunk " + _id(case), o, S, ro, rS, TOL[dt])


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129])
def test_chunk_ragged_tails(dev, T):
    inp = make(dev, 1, T, 2, 64, 32, torch.float32, seed=T, s0=0.05, b_scale=2.0)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    ro, rS = oracle(inp)
    check(f"chunk tail T={T}", o, S, ro, rS, 1e-4)


def _ws_sections(dk, dv, es, kb):
    a = lambda x: (x + 255) // 256 * 256
    kpad = (dk + kb - 1) // kb * kb
    qh = 0
    wwy = a(qh + 64 * kpad * es)
    ktt = a(wwy + 64 * kpad * es)
    p = a(ktt + dk * 64 * es)
    gaml = a(p + 64 * 64 * es)
    uwyt = a(gaml + dk * 4)
    block = a(uwyt + dv * 64 * es)
    return dict(qh=qh, wwy=wwy, ktt=ktt, p=p, gaml=gaml, uwyt=uwyt, block=block, kpad=kpad)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_chunk_prep_intermediates(dev, dt):
    """The workspace holds, per chunk, the oracle's chunked-form factors
    (Gamma*q, W = T(Gamma*b*k), Ktil, P, U = T(w*v), Gamma_L)."""
    B, T, H, dk, dv = 1, 100, 2, 64, 32
    inp = make(dev, B, T, H, dk, dv, dt, seed=5, b_scale=2.0)
    nbytes = g.chunk_prep_workspace_size(B, T, H, dk, dv, dt)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    g.chunk_prep(*args(inp), ws)
    torch.cuda.synchronize()
    h = {k_: _np(v_) for k_, v_ in inp.items() if v_ is not None}
    _, _, inter = chunked_wy(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], None, chunk=64,
                             return_intermediates=True)
    es = 4 if dt == torch.float32 else 2
    L = _ws_sections(dk, dv, es, 16 if es == 4 else 32)
    wsn = ws.cpu()
    nt = (T + 63) // 64
    tol = 1e-4 if dt == torch.float32 else 2e-2
    idx = 0
    for n in range(nt):
        for hi in range(H):
            ref = inter[idx]
            idx += 1
            Lc = ref["P"].shape[0]
            blk = wsn[((0 * H + hi) * nt + n) * L["block"]:((0 * H + hi) * nt + n + 1) * L["block"]]

            def sec(name, count, shape, dtype=dt):
                raw = blk[L[name]:L[name] + count * (4 if dtype == torch.float32 else 2)]
                return raw.view(dtype).float().numpy().reshape(shape)

            qh = sec("qh", 64 * L["kpad"], (64, L["kpad"]))[:Lc, :dk]
            wwy = sec("wwy", 64 * L["kpad"], (64, L["kpad"]))[:Lc, :dk]
            ktt = sec("ktt", dk * 64, (dk, 64))[:, :Lc]
            pm = sec("p", 64 * 64, (64, 64))
            gl = sec("gaml", dk, (dk,), torch.float32)
            ut = sec("uwyt", dv * 64, (dv, 64))[:, :Lc]
            for name, got, want in (("Qh", qh, ref["Qh"]), ("W", wwy, ref["W"]), ("Ktil^T", ktt, ref["Ktil"].T),
                                    ("P", pm[:Lc, :Lc], ref["P"]), ("U^T", ut, ref["U"].T),
                                    ("Gamma_L", gl, ref["GammaL"])):
                e = rel_l2(got, want)
                assert e <= tol, f"chunk {n} head {hi} {name}: rel-L2 {e:.3e}"
            # everything outside the valid rows/columns is exactly zero
            assert np.all(pm[:Lc, Lc:] == 0) and np.all(np.triu(pm[:Lc, :Lc], 1) == 0)
            if L["kpad"] > dk:
                assert np.all(sec("qh", 64 * L["kpad"], (64, L["kpad"]))[:, dk:] == 0)


def test_determinism(dev):
    inp = make(dev, 2, 300, 4, 128, 128, torch.bfloat16, seed=3, s0=0.05)
    o1, S1 = g.chunk_fwd(*args(inp), inp["S0"])
    o2, S2 = g.chunk_fwd(*args(inp), inp["S0"])
    r1, R1 = g.recurrent_step(*args(inp), inp["S0"])
    r2, R2 = g.recurrent_step(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert torch.equal(r1, r2) and torch.equal(R1, R2)


def test_split_resume(dev):
    """README "Quick start": the state returned by one call continues in the
    next.  A split at a chunk boundary reproduces the single call bit for bit;
    elsewhere it stays within tolerance of the oracle."""
    T = 300
    inp = make(dev, 2, T, 2, 128, 64, torch.bfloat16, seed=4, s0=0.05, b_scale=2.0)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    for t0 in (128, 100):
        part = lambda x, a_, b_: x[:, a_:b_].contiguous()
        a1 = [part(x, 0, t0) for x in args(inp)]
        a2 = [part(x, t0, T) for x in args(inp)]
        o1, S1 = g.chunk_fwd(*a1, inp["S0"])
        o2, S2 = g.chunk_fwd(*a2, S1)
        torch.cuda.synchronize()
        oc = torch.cat([o1, o2], dim=1)
        if t0 % 64 == 0:
            assert torch.equal(oc, o) and torch.equal(S2, S)
        ro, rS = oracle(inp)
        check(f"split at {t0}", oc, S2, ro, rS, 2e-2)
    # recurrent mode: any split is exact (same per-token arithmetic)
    r, R = g.recurrent_step(*args(inp), inp["S0"])
    a1 = [x[:, :77].contiguous() for x in args(inp)]
    a2 = [x[:, 77:].contiguous() for x in args(inp)]
    r1, R1 = g.recurrent_step(*a1, inp["S0"])
    r2, R2 = g.recurrent_step(*a2, R1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([r1, r2], 1), r) and torch.equal(R2, R)


def test_decode_in_place(dev):
    inp = make(dev, 8, 1, 4, 128, 128, torch.bfloat16, seed=9, s0=0.05)
    S = inp["S0"].clone()
    ro, rS = oracle(inp)
    o, S_ret = g.recurrent_step(*args(inp), S, inplace=True)
    torch.cuda.synchronize()
    assert S_ret.data_ptr() == S.data_ptr()
    check("decode in place", o, S, ro, rS, 2e-2)


def test_zero_state_default_and_empty(dev):
    inp = make(dev, 1, 80, 2, 64, 64, torch.bfloat16, seed=2)
    o1, S1 = g.chunk_fwd(*args(inp), None)
    o2, S2 = g.chunk_fwd(*args(inp), torch.zeros(1, 2, 64, 64, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    # T == 0: the state passes through unchanged, o is empty
    e = make(dev, 2, 0, 3, 32, 16, torch.float32, seed=1, s0=0.05)
    for fn in (g.chunk_fwd, g.recurrent_step):
        o, S = fn(*args(e), e["S0"])
        torch.cuda.synchronize()
        assert o.numel() == 0 and torch.equal(S, e["S0"])
        o, S = fn(*args(e), None)
        torch.cuda.synchronize()
        assert torch.count_nonzero(S) == 0
    # B == 0
    e = make(dev, 0, 10, 3, 32, 16, torch.bfloat16, seed=1)
    o, S = g.chunk_fwd(*args(e))
    assert o.shape == (0, 10, 3, 16) and S.shape == (0, 3, 32, 16)


def test_recall_invariant_gpu(dev):
    """Unit keys, b = 1, q = k: each output is exactly the gated value w*v
    (up to bf16 rounding), at any length and in both modes."""
    inp = make(dev, 2, 700, 4, 128, 128, torch.bfloat16, seed=6, s0=0.05)
    inp["q"] = inp["k"]
    inp["b"] = torch.ones_like(inp["b"])
    want = (inp["w"] * inp["v"].float()).cpu().numpy()
    for fn in (g.chunk_fwd, g.recurrent_step):
        o, _ = fn(*args(inp), inp["S0"])
        torch.cuda.synchronize()
        e = rel_l2(_np(o), want)
        print(f"[parity] recall {fn.__name__}: relL2 {e:.3e}", flush=True)
        assert e <= 2e-2


# ---------------------------------------------------------------------------
# full-size workloads, every chain, launched exactly as the benchmark does
# ---------------------------------------------------------------------------
def _full(dev, idx, seed):
    wl = inputs.WORKLOADS[idx]
    return wl, inputs.make(wl, seed, dev)


def test_full_chunk_B4_H16_T2048(dev):
    wl, inp = _full(dev, 1, seed=1)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    ro, rS = oracle(inp)
    check("full chunk B4 H16 T2048 (all 64 chains)", o, S, ro, rS, 2e-2)


def test_full_decode_B256_H16(dev):
    wl, inp = _full(dev, 2, seed=2)
    S = inp["S0"].clone()
    ro, rS = oracle(inp)
    o, _ = g.recurrent_step(*args(inp), S, inplace=True)
    torch.cuda.synchronize()
    check("full decode B256 H16 (all 4096 chains)", o, S, ro, rS, 2e-2)


def test_full_chunk_B1_H16_T65536(dev):
    wl, inp = _full(dev, 3, seed=3)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    ro, rS = oracle(inp)
    check("full chunk B1 H16 T65536 (all 16 chains)", o, S, ro, rS, 2e-2)


def test_full_chunk_B8_H16_T4096_dv256(dev):
    wl, inp = _full(dev, 4, seed=4)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    ro, rS = oracle(inp)
    check("full chunk B8 H16 T4096 dv256 (all 128 chains)", o, S, ro, rS, 2e-2)


# ---------------------------------------------------------------------------
# fast decay (alpha well below the workloads' sigmoid(N(3, 1))), both modes
# ---------------------------------------------------------------------------
FAST = [
    # B, T, H, dk, dv, dtype, alpha_mu, b scale
    (1, 300, 2, 128, 128, torch.bfloat16, 0.0, 2.0),
    (2, 257, 2, 128, 64, torch.bfloat16, -2.0, 1.0),
    (1, 200, 3, 64, 32, torch.float32, 0.0, 2.0),
    (1, 230, 2, 32, 48, torch.float32, -2.0, 2.0),
]


def _fid(c):
    B, T, H, dk, dv, dt, mu, bs = c
    return f"B{B}T{T}H{H}dk{dk}dv{dv}{'bf16' if dt == torch.bfloat16 else 'f32'}mu{mu:g}b{bs:g}"


@pytest.mark.parametrize("case", FAST, ids=_fid)
def test_fast_decay_both_modes(dev, case):
    B, T, H, dk, dv, dt, mu, bs = case
    inp = make(dev, B, T, H, dk, dv, dt, seed=T + 3, s0=0.05, b_scale=bs, alpha_mu=mu)
    ro, rS = oracle(inp)
    for fn in (g.chunk_fwd, g.recurrent_step):
        o, S = fn(*args(inp), inp["S0"])
        torch.cuda.synchronize()
        check(f"fast decay {fn.__name__} {_fid(case)}", o, S, ro, rS, TOL[dt])


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_decay_002_on_some_channels(dev, dt):
    """alpha = 0.02 on every fifth key channel for every token (the product over a
    16-token block is 0.02^16 = 6.6e-28), the workload's draw elsewhere."""
    B, T, H, dk, dv = 1, 260, 2, 128, 64
    inp = make(dev, B, T, H, dk, dv, dt, seed=41, s0=0.05, b_scale=2.0)
    inp["alpha"][..., ::5] = 0.02
    ro, rS = oracle(inp)
    for fn in (g.chunk_fwd, g.recurrent_step):
        o, S = fn(*args(inp), inp["S0"])
        torch.cuda.synchronize()
        check(f"alpha 0.02 on some channels {fn.__name__} {dt}", o, S, ro, rS, TOL[dt])


def test_tiny_fp32_workload_both_modes(dev):
    wl, inp = _full(dev, 0, seed=0)
    ro, rS = oracle(inp)
    for fn in (g.chunk_fwd, g.recurrent_step):
        o, S = fn(*args(inp), inp["S0"])
        torch.cuda.synchronize()
        check(f"tiny fp32 {fn.__name__}", o, S, ro, rS, 1e-4)


# ---------------------------------------------------------------------------
# the chunked forward at d128 bf16: tails, every value width, the stages
# called one by one, prologue options with grouped heads, decay extremes
# ---------------------------------------------------------------------------
def _split(inp, flags=0):
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, T, H, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    ws = g.alloc_workspace(g.chunk_prep_workspace_size(B, T, H, dk, dv, q.dtype, Hv=Hv), q.device)
    prob = g.problem(B, T, H, dk, dv, q.dtype, gate_dtype=inp["alpha"].dtype, flags=flags, Hv=Hv)
    g.chunk_prep(*args(inp), ws, flags=flags)
    o = torch.empty_like(v)
    S = torch.empty(B, Hv, dk, dv, dtype=torch.float32, device=q.device)
    g.chunk_state(prob, ws, o, inp["S0"], S)
    return o, S


FUSED = [
    # B, T, H, dk, dv, S0 std, b scale
    (1, 1, 2, 128, 128, 0.05, 1.0),
    (2, 63, 2, 128, 32, None, 2.0),
    (1, 64, 3, 128, 64, 0.05, 1.0),
    (1, 65, 2, 128, 96, 0.05, 2.0),
    (2, 129, 2, 128, 128, None, 1.0),
    (1, 300, 4, 128, 256, 0.05, 2.0),
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}dv{c[4]}{'S0' if c[5] else ''}b{c[6]:g}")
def test_chunk_d128_against_oracle_and_stages(dev, case):
    B, T, H, dk, dv, s0, bs = case
    inp = make(dev, B, T, H, dk, dv, torch.bfloat16, seed=T * 13 + dv, s0=s0, b_scale=bs)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    o2, S2 = _split(inp)
    torch.cuda.synchronize()
    ro, rS = oracle(inp)
    check(f"chunk_fwd B{B}T{T}H{H}dv{dv}", o, S, ro, rS, 2e-2)
    check(f"prep + state B{B}T{T}H{H}dv{dv}", o2, S2, ro, rS, 2e-2)


@pytest.mark.parametrize("mu", [-6.0, -12.0])
def test_chunk_decay_far_below_the_workloads(dev, mu):
    """alpha = sigmoid(N(mu, 1)): at mu = -12 the product over 16 tokens (~1e-83) is far
    outside the fp32 range; the chunked form's operands are bounded by products of 4 alphas
    (~1e-21) and it stays at the bf16 bar in both output and state."""
    inp = make(dev, 2, 200, 2, 128, 64, torch.bfloat16, seed=int(-mu) + 50, s0=0.05, b_scale=2.0,
               alpha_mu=mu)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    ro, rS = oracle(inp)
    check(f"chunk alpha_mu {mu}", o, S, ro, rS, 2e-2)


def test_chunk_decay_fp32_far_below(dev):
    """The fp32 operand path (dk 64, dv 48) at alpha = sigmoid(N(-8, 1)), against the fp32 bar."""
    inp = make(dev, 1, 230, 2, 64, 48, torch.float32, seed=71, s0=0.05, b_scale=2.0, alpha_mu=-8.0)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    ro, rS = oracle(inp)
    check("chunk fp32 alpha_mu -8", o, S, ro, rS, 1e-4)


def test_chunk_decay_mix_and_exact_one(dev):
    """alpha = 1 exactly on some channels (no decay), 1e-3 on others, the draw elsewhere."""
    inp = make(dev, 1, 260, 3, 128, 128, torch.bfloat16, seed=61, s0=0.05, b_scale=2.0)
    inp["alpha"][..., ::7] = 1.0
    inp["alpha"][..., 3::7] = 1e-3
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    ro, rS = oracle(inp)
    check("chunk alpha mix", o, S, ro, rS, 2e-2)


@pytest.mark.parametrize("flags", [1, 3, 4, 7])
def test_chunk_d128_prologue_flags_and_grouped_heads(dev, flags):
    """In-kernel prologue (gate logits in bf16, b x 2, q/k L2 norm) and 2 value heads per
    query/key head at d128, against the oracle with the same options."""
    from oracle.reference import share_qk_heads
    B, T, H, Hv, dk, dv = 2, 150, 2, 4, 128, 64
    inp = inputs.make_raw(B, T, H, dk, dv, torch.bfloat16, 70 + flags, dev, s0_std=0.05, Hv=Hv,
                          gate_logits=bool(flags & 1), unit_qk=not flags & 4,
                          gate_dtype=torch.bfloat16 if flags & 1 else torch.float32)
    o, S = g.chunk_fwd(*args(inp), inp["S0"], flags=flags)
    o2, S2 = _split(inp, flags)
    torch.cuda.synchronize()
    h = {k_: _np(v_) for k_, v_ in inp.items()}
    qw, kw = share_qk_heads(h["q"], h["k"], Hv)
    ro, rS = c_oracle.recurrent(qw, kw, h["v"], h["alpha"], h["b"], h["w"], h["S0"], flags=flags)
    check(f"chunk_fwd flags {flags} Hv {Hv}", o, S, ro, rS, 2e-2)
    check(f"prep + state flags {flags} Hv {Hv}", o2, S2, ro, rS, 2e-2)


def test_chunk_d128_split_resume_bitwise(dev):
    """Two calls split at a chunk boundary equal one call bit for bit (the state crosses
    the boundary in fp32 either way), and the state may be updated in place."""
    T = 320
    inp = make(dev, 1, T, 4, 128, 128, torch.bfloat16, seed=88, s0=0.05, b_scale=2.0)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    a1 = [x[:, :192].contiguous() for x in args(inp)]
    a2 = [x[:, 192:].contiguous() for x in args(inp)]
    o1, S1 = g.chunk_fwd(*a1, inp["S0"])
    o2, S2 = g.chunk_fwd(*a2, S1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], 1), o) and torch.equal(S2, S)
    # in place: S_out == S0
    Sp = inp["S0"].clone()
    o3, _ = g.chunk_fwd(*args(inp), Sp, S_out=Sp)
    torch.cuda.synchronize()
    assert torch.equal(o3, o) and torch.equal(Sp, S)


# ---------------------------------------------------------------------------
# a long single sequence with few chains runs in pieces (the prep of later
# pieces on a second stream beside the state pass); chunk boundaries are
# bitwise resumable, so the pieces must equal the two stages called once
# ---------------------------------------------------------------------------
PIECES = [
    # T, H, Hv, dk, dv, dtype, gate dtype, flags, S0 std
    (256 * 64 + 37, 2, 2, 64, 64, torch.float32, torch.float32, 0, 0.05),
    (300 * 64, 1, 2, 128, 128, torch.bfloat16, torch.bfloat16,
     g.FLAG_GATE_LOGITS | g.FLAG_NEG_EIGVAL | g.FLAG_QK_L2NORM, None),
    (1024 * 64 + 1, 2, 2, 128, 128, torch.bfloat16, torch.float32, 0, 0.05),
    (256 * 64 + 9, 1, 1, 128, 256, torch.bfloat16, torch.float32, 0, 0.05),
    (384 * 64 + 63, 3, 3, 64, 128, torch.bfloat16, torch.float32, 0, 0.05),
    (256 * 64 + 17, 2, 2, 64, 64, torch.bfloat16, torch.float32, 0, 0.05),
]


@pytest.mark.parametrize("case", PIECES, ids=lambda c: f"T{c[0]}H{c[1]}Hv{c[2]}dk{c[3]}dv{c[4]}fl{c[7]}")
def test_long_sequence_in_pieces(dev, case):
    T, H, Hv, dk, dv, dt, gt, flags, s0 = case
    print(f"pieces T={T} H={H} Hv={Hv} dk={dk} dv={dv} {dt} flags {flags}", flush=True)
    inp = inputs.make_raw(1, T, H, dk, dv, dt, 61 + dk, dev, s0_std=s0, Hv=Hv, gate_dtype=gt,
                          gate_logits=bool(flags & g.FLAG_GATE_LOGITS), unit_qk=not flags & g.FLAG_QK_L2NORM)
    o, S = g.chunk_fwd(*args(inp), inp["S0"], flags=flags)
    o2, S2 = _split(inp, flags)
    # in place: S_out is the initial state's buffer
    S_io = inp["S0"].clone() if inp["S0"] is not None else None
    o3 = torch.empty_like(o)
    if S_io is not None:
        g.chunk_fwd(*args(inp), S_io, flags=flags, o=o3, S_out=S_io)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2), "pieces differ from the single pass"
    if S_io is not None:
        assert torch.equal(o3, o) and torch.equal(S_io, S), "in-place pieces differ"
    if T <= 300 * 64:
        from oracle.reference import share_qk_heads
        f = lambda x: None if x is None else x.detach().to("cpu", torch.float32).numpy()
        qq, kk = f(inp["q"]), f(inp["k"])
        if Hv != H:
            qq, kk = (np.ascontiguousarray(x, dtype=np.float32) for x in share_qk_heads(qq, kk, Hv))
        ro, rS = c_oracle.recurrent(qq, kk, f(inp["v"]), f(inp["alpha"]), f(inp["b"]), f(inp["w"]), f(inp["S0"]),
                                    flags=flags)
        check(f"pieces T{T}", o, S, ro, rS, 1e-4 if dt == torch.float32 else 2e-2)


def test_long_sequence_under_graph_capture(dev):
    """A forward that runs in pieces when called eagerly (second stream) is captured into a
    graph as one stream's work; replays, with eager work and synchronisations between them,
    equal the eager result bit for bit."""
    T, H, dk, dv = 256 * 64 + 5, 2, 64, 64
    inp = inputs.make_raw(1, T, H, dk, dv, torch.bfloat16, 71, dev, s0_std=0.05)
    o_ref, S_ref = g.chunk_fwd(*args(inp), inp["S0"])
    ws = g.alloc_workspace(g.chunk_fwd_workspace_size(1, T, H, dk, dv, torch.bfloat16), dev)
    o = torch.empty_like(o_ref)
    S = torch.empty_like(S_ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.chunk_fwd(*args(inp), inp["S0"], o=o, S_out=S, workspace=ws)
    for rep in range(4):
        o.zero_()
        S.fill_(1.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), f"replay {rep}"
        g.chunk_fwd(*args(inp), inp["S0"], o=torch.empty_like(o), workspace=ws)   # eager work between replays
        torch.cuda.synchronize()
