"""GPU parity of the HIP path against the fp64 CPU oracle (needs an MI355X).

Every comparison feeds both sides the same seeded inputs (bf16 inputs are
widened exactly for the oracle) and measures the relative L2 error over the
whole tensor, for o and for the final state separately:
    <= 1e-4 for fp32 I/O, <= 2e-2 for bf16 I/O with the fp32 state.
Full-size workloads are compared on sampled (batch, head) chains, which the
recurrence keeps independent, with the GPU run in exactly the launch
configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as g
from gated_delta_rule_19_amd import inputs
from oracle import c_oracle
from oracle.reference import chunked_wy, rel_l2

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


def check(what, o, S, ref_o, ref_S, tol):
    eo = rel_l2(_np(o) if torch.is_tensor(o) else o, ref_o)
    eS = rel_l2(_np(S) if torch.is_tensor(S) else S, ref_S)
    print(f"[parity] {what}: relL2 o={eo:.3e} S={eS:.3e} (tol {tol:g})", flush=True)
    assert eo <= tol, f"{what}: o rel-L2 {eo:.3e} > {tol}"
    assert eS <= tol, f"{what}: S rel-L2 {eS:.3e} > {tol}"


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
    nbytes = g.chunk_fwd_workspace_size(B, T, H, dk, dv, dt)
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
# full-size workloads (sampled chains), launched exactly as the benchmark does
# ---------------------------------------------------------------------------
def _full(dev, idx, seed):
    wl = inputs.WORKLOADS[idx]
    return wl, inputs.make(wl, seed, dev)


def test_full_chunk_B4_H16_T2048(dev):
    wl, inp = _full(dev, 1, seed=1)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    chains = [(0, 0), (1, 7), (2, 11), (3, 15)]
    ro, rS = oracle(inp, chains=chains)
    go, gS = pick(o, S, chains)
    check("full chunk B4 H16 T2048 (4 heads)", go, gS, ro, rS, 2e-2)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()


def test_full_decode_B256_H16(dev):
    wl, inp = _full(dev, 2, seed=2)
    S = inp["S0"].clone()
    ro, rS = oracle(inp)
    o, _ = g.recurrent_step(*args(inp), S, inplace=True)
    torch.cuda.synchronize()
    check("full decode B256 H16 (all heads)", o, S, ro, rS, 2e-2)


def test_full_chunk_B1_H16_T65536(dev):
    wl, inp = _full(dev, 3, seed=3)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    chains = [(0, 5)]
    ro, rS = oracle(inp, chains=chains)
    go, gS = pick(o, S, chains)
    check("full chunk B1 H16 T65536 (1 head)", go, gS, ro, rS, 2e-2)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()


def test_full_chunk_B8_H16_T4096_dv256(dev):
    wl, inp = _full(dev, 4, seed=4)
    o, S = g.chunk_fwd(*args(inp), inp["S0"])
    torch.cuda.synchronize()
    chains = [(0, 3), (7, 12)]
    ro, rS = oracle(inp, chains=chains)
    go, gS = pick(o, S, chains)
    check("full chunk B8 H16 T4096 dv256 (2 heads)", go, gS, ro, rS, 2e-2)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()


def test_tiny_fp32_workload_both_modes(dev):
    wl, inp = _full(dev, 0, seed=0)
    ro, rS = oracle(inp)
    for fn in (g.chunk_fwd, g.recurrent_step):
        o, S = fn(*args(inp), inp["S0"])
        torch.cuda.synchronize()
        check(f"tiny fp32 {fn.__name__}", o, S, ro, rS, 1e-4)
