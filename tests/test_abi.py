"""C-ABI contract checks that need no GPU (include/gdn2.h).

The library loads on a host without a GPU (it only links the HIP runtime);
every argument check runs on the host before any HIP call, so each error path
is exercised here with fake device addresses that are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_19_amd as g
from gated_delta_rule_19_amd import _binding as bnd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn2.h")

OK, NULL, SHAPE, DTYPE, ALIAS, WS, DEVICE, ALIGN = range(8)
BASE = 0x7f0000000000          # fake, 256-aligned, never dereferenced


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(gdn2_\w+)\s*\(", src, re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(bnd.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", bnd.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(gdn2_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(g.lib(), name)


def test_version_and_status_strings():
    assert g.abi_version() == 8
    for code in range(8):
        assert g.status_str(code).startswith(bnd._STATUS[code])
    assert "unknown" in g.status_str(99)


def test_problem_struct_layout():
    assert ctypes.sizeof(bnd.Problem) == 64
    assert bnd.Problem.Hv.offset == 56


class Call:
    """Lay out fake, disjoint device buffers for one problem."""

    def __init__(self, B=2, T=100, H=3, dk=64, dv=32, io=1, gate=0, chunk=64, flags=0, Hv=0):
        self.p = bnd.Problem(B, T, H, dk, dv, chunk, io, gate, flags, Hv)
        es = 2 if io == 1 else 4
        gs = 2 if gate == 1 else 4
        rows, vrows, nv = B * T * H, B * T * (Hv or H), B * (Hv or H)
        sizes = dict(q=rows * dk * es, k=rows * dk * es, v=vrows * dv * es, alpha=vrows * dk * gs,
                     b=vrows * dk * gs, w=vrows * dv * gs, S0=nv * dk * dv * 4, o=vrows * dv * es,
                     S_out=nv * dk * dv * 4)
        sizes["ws"] = g.lib().gdn2_chunk_prep_workspace_size(ctypes.byref(self.p)) or 256
        self.size = sizes
        addr = BASE
        self.ptr = {}
        for name, n in sizes.items():
            self.ptr[name] = addr
            addr += (n + 4095) // 4096 * 4096 + 4096

    def fwd(self, **over):
        a = dict(self.ptr)
        a.update(over)
        P = lambda x: None if x is None else ctypes.c_void_p(x)
        wsb = over.pop("ws_bytes", None) if "ws_bytes" in over else self.size["ws"]
        return g.lib().gdn2_chunk_fwd(ctypes.byref(self.p), *(P(a[n]) for n in
                                      ("q", "k", "v", "alpha", "b", "w", "S0", "o", "S_out")),
                                      P(a["ws"]), wsb, None)

    def rec(self, **over):
        a = dict(self.ptr)
        a.update(over)
        P = lambda x: None if x is None else ctypes.c_void_p(x)
        return g.lib().gdn2_recurrent_step(ctypes.byref(self.p), *(P(a[n]) for n in
                                           ("q", "k", "v", "alpha", "b", "w", "S0", "o", "S_out")), None)


def test_valid_call_reaches_the_device_check():
    # on a host with no GPU the first HIP call fails -> GDN2_ERR_DEVICE
    c = Call()
    assert c.fwd() == DEVICE
    assert c.rec() == DEVICE


def test_workspace_size():
    torch = __import__("torch")
    p = bnd.problem(4, 2048, 16, 128, 128, torch.bfloat16)
    # one 256-aligned block per (batch, head, chunk); bf16 block = 74,240 bytes at dk = dv = 128
    assert g.lib().gdn2_chunk_fwd_workspace_size(ctypes.byref(p)) == 4 * 16 * 32 * 74240
    # the stages on their own need the same
    for shape in ((4, 2048, 16, 128, 128, torch.bfloat16), (4, 2048, 16, 64, 64, torch.bfloat16),
                  (1, 100, 2, 128, 128, torch.float32), (1, 100, 2, 128, 48, torch.bfloat16)):
        p2 = bnd.problem(*shape)
        n = g.lib().gdn2_chunk_fwd_workspace_size(ctypes.byref(p2))
        assert n == g.lib().gdn2_chunk_prep_workspace_size(ctypes.byref(p2)) > 0
    assert g.lib().gdn2_chunk_fwd_workspace_size(None) == 0
    assert g.lib().gdn2_chunk_prep_workspace_size(None) == 0
    bad = bnd.Problem(1, 1, 1, 100, 16, 64, 1, 0, 0)
    assert g.lib().gdn2_chunk_fwd_workspace_size(ctypes.byref(bad)) == 0


@pytest.mark.parametrize("field,value", [("dk", 48), ("dk", 256), ("dv", 8), ("dv", 24), ("dv", 272),
                                         ("B", -1), ("T", -1), ("chunk", 32), ("flags", 8), ("flags", 2),
                                         ("flags", 6), ("flags", -1)])
def test_shape_errors(field, value):
    c = Call()
    setattr(c.p, field, value)
    if field == "chunk":
        assert c.fwd() == SHAPE and c.rec() == DEVICE   # the recurrent mode ignores chunk
    else:
        assert c.fwd() == SHAPE and c.rec() == SHAPE


@pytest.mark.parametrize("io,gate", [(0, 1), (2, 0), (1, 5), (1, 2)])
def test_dtype_errors(io, gate):
    c = Call(io=io, gate=gate)
    assert c.fwd() == DTYPE and c.rec() == DTYPE


@pytest.mark.parametrize("io,gate,flags", [(0, 0, 0), (1, 0, 0), (1, 1, 0), (1, 1, 1), (1, 1, 3), (1, 0, 4),
                                           (0, 0, 7), (1, 1, 5)])
def test_supported_dtypes_and_flags_reach_the_device_check(io, gate, flags):
    c = Call(io=io, gate=gate, flags=flags)
    assert c.fwd() == DEVICE and c.rec() == DEVICE


def test_bf16_gates_are_sized_as_bf16():
    # one token, dk = 64: alpha holds 128 bytes in bf16 (256 in fp32); a state
    # placed right after those 128 bytes overlaps nothing
    c = Call(B=1, T=1, H=1, dk=64, dv=16, io=1, gate=1)
    assert c.fwd(S_out=c.ptr["alpha"] + 128) == DEVICE
    assert c.fwd(S_out=c.ptr["alpha"] + 112) == ALIAS
    f = Call(B=1, T=1, H=1, dk=64, dv=16, io=1, gate=0)
    assert f.fwd(S_out=f.ptr["alpha"] + 128) == ALIAS


@pytest.mark.parametrize("H,Hv,want", [(3, 0, DEVICE), (3, 3, DEVICE), (3, 6, DEVICE), (2, 8, DEVICE),
                                       (1, 16, DEVICE), (3, 4, SHAPE), (4, 2, SHAPE), (3, -3, SHAPE),
                                       (0, 2, SHAPE)])
def test_value_head_counts(H, Hv, want):
    c = Call(H=H, Hv=Hv)
    assert c.fwd() == want and c.rec() == want


def test_grouped_heads_are_sized_per_tensor():
    # B = T = 1, H = 1 query/key head of dk = 64 (128 bytes bf16), Hv = 4 value
    # heads: v is 4 x 16 bf16 = 128 bytes, the state 4 x 64 x 16 fp32
    c = Call(B=1, T=1, H=1, Hv=4, dk=64, dv=16, io=1, gate=1)
    assert c.fwd(o=c.ptr["q"] + 128) == DEVICE          # q holds one head only
    assert c.fwd(o=c.ptr["v"] + 112) == ALIAS           # v holds all four
    assert c.fwd(o=c.ptr["alpha"] + 496) == ALIAS       # alpha: 4 x 64 bf16 = 512 bytes
    assert c.fwd(o=c.ptr["alpha"] + 512) == DEVICE
    one = bnd.problem(2, 300, 4, 128, 128, __import__("torch").bfloat16)
    four = bnd.problem(2, 300, 4, 128, 128, __import__("torch").bfloat16, Hv=16)
    ws = lambda p: g.lib().gdn2_chunk_prep_workspace_size(ctypes.byref(p))
    assert ws(four) == 4 * ws(one) > 0                  # one workspace block per value head and chunk


def test_null_errors():
    c = Call()
    assert g.lib().gdn2_chunk_fwd(None, *([None] * 10), 0, None) == NULL
    for name in ("q", "k", "v", "alpha", "b", "w", "o"):
        assert c.fwd(**{name: None}) == NULL, name
        assert c.rec(**{name: None}) == NULL, name
    # S0 and S_out are optional
    assert c.fwd(S0=None, S_out=None) == DEVICE
    assert c.rec(S0=None) == DEVICE


def test_empty_problems_need_no_pointers_and_no_device():
    for B, T, H in ((0, 10, 2), (2, 10, 0)):
        c = Call(B=B, T=T, H=H)
        none = {n: None for n in ("q", "k", "v", "alpha", "b", "w", "S0", "o", "S_out", "ws")}
        assert c.fwd(**none, ws_bytes=0) == OK
        assert c.rec(**none) == OK
    # T == 0 with the state updated in place is a no-op
    c = Call(T=0)
    assert c.rec(q=None, k=None, v=None, alpha=None, b=None, w=None, o=None, S_out=c.ptr["S0"]) == OK
    assert c.fwd(q=None, k=None, v=None, alpha=None, b=None, w=None, o=None, ws=None, ws_bytes=0,
                 S_out=c.ptr["S0"]) == OK


def test_workspace_errors():
    c = Call()
    assert c.fwd(ws=None) == WS
    assert c.fwd(ws_bytes=c.size["ws"] - 1) == WS
    assert c.fwd(ws=c.ptr["ws"] + 16) == WS        # not 256-byte aligned


def test_alias_errors():
    c = Call()
    # an output overlapping an input
    assert c.fwd(o=c.ptr["q"] + 64) == ALIAS
    assert c.rec(o=c.ptr["v"]) == ALIAS
    assert c.fwd(S_out=c.ptr["alpha"]) == ALIAS
    assert c.fwd(ws=c.ptr["w"]) == ALIAS
    # outputs overlapping each other
    assert c.fwd(S_out=c.ptr["o"]) == ALIAS
    assert c.fwd(ws=c.ptr["o"]) == ALIAS
    # the state may be updated in place only with identical pointers
    assert c.fwd(S_out=c.ptr["S0"]) == DEVICE
    assert c.rec(S_out=c.ptr["S0"]) == DEVICE
    assert c.fwd(S_out=c.ptr["S0"] + 256) == ALIAS
    assert c.rec(S_out=c.ptr["S0"] + 4) == ALIAS


def test_alignment_errors():
    c = Call()
    for name in ("q", "k", "v", "alpha", "b", "w", "o", "S_out", "S0"):
        assert c.fwd(**{name: c.ptr[name] + 8}) == ALIGN, name
        assert c.rec(**{name: c.ptr[name] + 4}) == ALIGN, name


def test_stage_entry_points_validate():
    c = Call()
    P = ctypes.c_void_p
    L = g.lib()
    args = [P(c.ptr[n]) for n in ("q", "k", "v", "alpha", "b", "w")]
    assert L.gdn2_chunk_prep(ctypes.byref(c.p), *args, P(c.ptr["ws"]), c.size["ws"], None) == DEVICE
    assert L.gdn2_chunk_prep(ctypes.byref(c.p), *args, None, c.size["ws"], None) == WS
    assert L.gdn2_chunk_prep(ctypes.byref(c.p), *args, P(c.ptr["q"]), c.size["ws"], None) == ALIAS
    assert L.gdn2_chunk_state(ctypes.byref(c.p), P(c.ptr["S0"]), P(c.ptr["o"]), P(c.ptr["S_out"]),
                              P(c.ptr["ws"]), c.size["ws"], None) == DEVICE
    assert L.gdn2_chunk_state(ctypes.byref(c.p), None, None, None, P(c.ptr["ws"]), c.size["ws"], None) == NULL
    assert L.gdn2_chunk_state(ctypes.byref(c.p), None, P(c.ptr["ws"]), None, P(c.ptr["ws"]),
                              c.size["ws"], None) == ALIAS


def test_binding_rejects_cpu_tensors_and_bad_shapes():
    import torch
    q = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        g.recurrent_step(q, q, torch.zeros(1, 4, 1, 16), q, q, torch.zeros(1, 4, 1, 16))
    with pytest.raises(ValueError):
        g.chunk_fwd(q, q, torch.zeros(1, 4, 2, 16), q, q, torch.zeros(1, 4, 2, 16))
    with pytest.raises(TypeError):
        g.chunk_fwd(q.double(), q.double(), torch.zeros(1, 4, 1, 16).double(), q, q, torch.zeros(1, 4, 1, 16))


def test_gated_rmsnorm_validates():
    c = Call(B=2, T=10, H=3, dk=64, dv=48)
    L = g.lib()
    P = ctypes.c_void_p
    o, gt, y = c.ptr["o"], c.ptr["v"], c.ptr["S_out"]
    wt = c.ptr["w"]
    call = lambda **kw: L.gdn2_gated_rmsnorm(ctypes.byref(c.p), *(P(kw.get(n, d)) if kw.get(n, d) is not None
                                                                  else None for n, d in
                                                                  (("o", o), ("g", gt), ("wt", wt), ("y", y))),
                                             None)
    assert call() == DEVICE
    assert call(y=o) == DEVICE                  # in place
    assert call(y=o + 16) == ALIAS
    assert call(y=gt) == ALIAS
    assert call(g=None) == NULL and call(wt=None) == NULL and call(y=None) == NULL
    assert call(o=o + 8) == ALIGN
    empty = Call(B=0)
    assert L.gdn2_gated_rmsnorm(ctypes.byref(empty.p), None, None, None, None, None) == OK
    bad = Call(dv=40)
    assert L.gdn2_gated_rmsnorm(ctypes.byref(bad.p), P(o), P(gt), P(wt), P(y), None) == SHAPE


class VCall(Call):
    """Fake buffers of a packed batch: N sequences, T packed tokens."""

    def __init__(self, N=3, T=100, H=2, dk=64, dv=32, io=1, gate=0, flags=0, Hv=0):
        super().__init__(B=1, T=T, H=H, dk=dk, dv=dv, io=io, gate=gate, flags=flags, Hv=Hv)
        self.p.B = N
        nv = N * (Hv or H)
        self.size["S0"] = self.size["S_out"] = nv * dk * dv * 4
        self.size["cu"] = 4 * (N + 1)
        self.size["ws"] = g.lib().gdn2_chunk_fwd_varlen_workspace_size(ctypes.byref(self.p)) or 256
        addr = BASE
        for name, n in self.size.items():
            self.ptr[name] = addr
            addr += (n + 4095) // 4096 * 4096 + 4096

    def fwd(self, **over):
        a = dict(self.ptr)
        a.update(over)
        P = lambda x: None if x is None else ctypes.c_void_p(x)
        wsb = over.pop("ws_bytes", None) if "ws_bytes" in over else self.size["ws"]
        return g.lib().gdn2_chunk_fwd_varlen(ctypes.byref(self.p), P(a["cu"]), *(P(a[n]) for n in
                                             ("q", "k", "v", "alpha", "b", "w", "S0", "o", "S_out")),
                                             P(a["ws"]), wsb, None)

    def rec(self, **over):
        a = dict(self.ptr)
        a.update(over)
        P = lambda x: None if x is None else ctypes.c_void_p(x)
        return g.lib().gdn2_recurrent_varlen(ctypes.byref(self.p), P(a["cu"]), *(P(a[n]) for n in
                                             ("q", "k", "v", "alpha", "b", "w", "S0", "o", "S_out")), None)


def test_varlen_valid_calls_reach_the_device_check():
    for kw in ({}, {"Hv": 4}, {"io": 0}, {"gate": 1, "flags": 7}, {"N": 1}, {"T": 0}):
        c = VCall(**kw)
        assert c.fwd() == DEVICE and c.rec() == DEVICE, kw


def test_varlen_workspace_size():
    # plan (2 (N+1) int32 offsets + 8 bytes per chunk slot, 256-aligned), then one
    # block per (value head, chunk slot); slots = ceil(T / 64) + N
    import torch
    N, T, H, Hv = 5, 1000, 4, 8
    p = bnd.problem(N, T, H, 128, 128, torch.bfloat16, Hv=Hv)
    slots = (T + 63) // 64 + N
    plan = (4 * 2 * (N + 1) + 8 * slots + 255) // 256 * 256
    assert g.lib().gdn2_chunk_fwd_varlen_workspace_size(ctypes.byref(p)) == plan + Hv * slots * 74240
    bad = bnd.problem(N, T, H, 100, 128, torch.bfloat16)
    assert g.lib().gdn2_chunk_fwd_varlen_workspace_size(ctypes.byref(bad)) == 0


def test_varlen_errors():
    c = VCall()
    assert c.fwd(cu=None) == NULL and c.rec(cu=None) == NULL
    assert c.fwd(cu=c.ptr["cu"] + 2) == ALIGN and c.rec(cu=c.ptr["cu"] + 2) == ALIGN
    assert c.fwd(cu=c.ptr["cu"] + 4) == DEVICE                  # int32 alignment is enough
    assert c.fwd(o=c.ptr["cu"]) == ALIAS and c.rec(S_out=c.ptr["cu"]) == ALIAS
    assert c.fwd(ws=c.ptr["cu"]) == ALIAS
    assert c.fwd(ws_bytes=c.size["ws"] - 1) == WS and c.fwd(ws=None) == WS
    assert c.fwd(q=None) == NULL and c.rec(w=None) == NULL
    assert c.fwd(S_out=c.ptr["S0"]) == DEVICE and c.rec(S_out=c.ptr["S0"]) == DEVICE   # in place
    assert c.fwd(S_out=c.ptr["S0"] + 256) == ALIAS
    big = VCall(T=2 ** 31 - 60)
    assert big.fwd() == SHAPE and big.rec() == SHAPE
    chunk = VCall()
    chunk.p.chunk = 32
    assert chunk.fwd() == SHAPE and chunk.rec() == DEVICE


def test_varlen_states_are_per_sequence():
    # N = 3 sequences, Hv = 4, dk = 64, dv = 32: a state tensor holds 3 x 4 x 64 x 32 fp32
    c = VCall(N=3, Hv=4)
    n = 3 * 4 * 64 * 32 * 4
    assert c.fwd(o=c.ptr["S0"] + n) == DEVICE
    assert c.fwd(o=c.ptr["S0"] + n - 256) == ALIAS


def test_varlen_empty_calls_need_no_pointers():
    none = {n: None for n in ("cu", "q", "k", "v", "alpha", "b", "w", "S0", "o", "S_out", "ws")}
    c = VCall(N=0)
    assert c.fwd(**none, ws_bytes=0) == OK and c.rec(**none) == OK
    # no tokens and the state left in place: nothing to do
    t0 = VCall(T=0)
    assert t0.fwd(q=None, k=None, v=None, alpha=None, b=None, w=None, o=None, S_out=t0.ptr["S0"]) == OK
    assert t0.rec(q=None, k=None, v=None, alpha=None, b=None, w=None, o=None, S_out=t0.ptr["S0"]) == OK


def test_varlen_binding_validates():
    import torch
    q = torch.zeros(1, 8, 2, 16)
    v = torch.zeros(1, 8, 2, 16)
    cu = torch.tensor([0, 3, 8], dtype=torch.int32)
    with pytest.raises(ValueError):          # CPU tensors
        g.chunk_fwd_varlen(q, q, v, q, q, v, cu)
    with pytest.raises(ValueError):
        g.recurrent_varlen(q, q, v, q, q, v, cu.long())


# ---- backward ----------------------------------------------------------------------
def _up(x):
    return (x + 255) // 256 * 256


def _bwd_ws(B, T, H, dk, dv, io, gate, flags, Hv):
    return g.lib().gdn2_chunk_bwd_workspace_size(ctypes.byref(bnd.Problem(B, T, H, dk, dv, 64, io, gate, flags, Hv)))


@pytest.mark.parametrize("flags,Hv,gate,dv", [(0, 0, 0, 32), (4, 0, 1, 32), (1, 0, 1, 32), (3, 6, 0, 32),
                                                (0, 6, 1, 32), (7, 6, 1, 32), (7, 0, 1, 48), (4, 0, 0, 48)])
def test_backward_workspace_with_options(flags, Hv, gate, dv):
    """The matrix-core path (bf16 I/O, dk and dv in {32, 64, 128}) applies the prologue
    options in-kernel: with one value head per query/key head its workspace is the plain
    one.  Otherwise (shared query/key heads, or the vector-ALU path) the workspace is the
    core's (no flags, one query/key head per value head, fp32 gates with logits) followed
    by 256-aligned activated inputs and their gradients."""
    B, T, H, dk, io = 2, 100, 3, 64, 1
    hv = Hv or H
    mf = dv in (32, 64, 128)
    if mf and hv == H:
        assert _bwd_ws(B, T, H, dk, dv, io, gate, flags, Hv) == _bwd_ws(B, T, H, dk, dv, io, gate, 0, 0)
        return
    gates_mapped = flags & 1 and not mf         # the matrix-core kernels take gate logits themselves
    core = _bwd_ws(B, T, hv, dk, dv, io, 0 if gates_mapped else gate, 0, 0)
    assert core > 0
    off = core
    parts = []
    vrows = B * T * hv
    if flags & 4 or hv != H:
        parts += [vrows * dk * 2] * 4
    if gates_mapped:
        parts += [vrows * dk * 4, vrows * dk * 4, vrows * dv * 4] * 2
    for n in parts:
        off = _up(off) + n
    assert _bwd_ws(B, T, H, dk, dv, io, gate, flags, Hv) == off


class BCall:
    """Fake, disjoint device buffers for one backward call."""

    def __init__(self, B=2, T=100, H=3, dk=64, dv=32, io=1, gate=0, flags=0, Hv=0):
        self.p = bnd.Problem(B, T, H, dk, dv, 64, io, gate, flags, Hv)
        es, gs = (2 if io == 1 else 4), (2 if gate == 1 else 4)
        rows, vrows, nv = B * T * H, B * T * (Hv or H), B * (Hv or H)
        st = nv * dk * dv * 4
        self.names = ("q", "k", "v", "alpha", "b", "w", "S0", "dO", "dS_T", "dq", "dk", "dv", "dalpha", "db",
                      "dw", "dS0", "ws")
        sz = dict(q=rows * dk * es, k=rows * dk * es, v=vrows * dv * es, alpha=vrows * dk * gs, b=vrows * dk * gs,
                  w=vrows * dv * gs, S0=st, dO=vrows * dv * es, dS_T=st)
        for n in ("q", "k", "v", "alpha", "b", "w"):
            sz["d" + n] = sz[n]
        sz["dS0"] = st
        sz["ws"] = g.lib().gdn2_chunk_bwd_workspace_size(ctypes.byref(self.p))
        self.size, self.ptr, addr = sz, {}, BASE
        for n in self.names:
            self.ptr[n] = addr
            addr += (sz[n] + 4095) // 4096 * 4096 + 4096

    def __call__(self, **over):
        wsb = over.pop("ws_bytes", self.size["ws"])
        a = dict(self.ptr)
        a.update(over)
        P = lambda x: None if x is None else ctypes.c_void_p(x)
        return g.lib().gdn2_chunk_bwd(ctypes.byref(self.p), *(P(a[n]) for n in self.names), wsb, None)


@pytest.mark.parametrize("flags,Hv", [(0, 0), (7, 0), (4, 6), (1, 3)])
def test_backward_checks(flags, Hv):
    c = BCall(flags=flags, Hv=Hv)
    assert c.size["ws"] > 0
    assert c() == DEVICE
    assert c(ws_bytes=c.size["ws"] - 1) == WS
    assert c(ws=c.ptr["ws"] + 16) == WS
    assert c(dq=None) == NULL
    assert c(dq=c.ptr["q"]) == ALIAS
    assert c(ws=c.ptr["dalpha"]) == ALIAS
    assert c(dS0=c.ptr["S0"]) == ALIAS           # no in-place state gradient
    assert c(dalpha=c.ptr["dalpha"] + 8) == ALIGN
    assert c(S0=None, dS_T=None, dS0=None) == DEVICE


def test_backward_rejects_what_the_forward_rejects():
    assert BCall(flags=2).__call__() == SHAPE     # negative eigenvalues need gate logits
    assert BCall(Hv=4).__call__() == SHAPE        # 4 value heads over 3 query/key heads
    assert _bwd_ws(2, 100, 3, 64, 32, 1, 0, 2, 0) == 0
